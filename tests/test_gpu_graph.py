"""The whole layer captured in a HIP graph: every replay equals the eager
result bit for bit, with eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_wave_amd as moe
from synth import CONFIGS, generate

from gpu_helpers import BF16_TOL, clear_tokens, max_rel_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()


@pytest.mark.parametrize("T,d,d_ff", [(4, 512, 1024), (1, 512, 512), (300, 256, 384)])
def test_graph_replay_matches_eager(T, d, d_ff):
    say(f"graph replay T={T} d={d} d_ff={d_ff}")
    cfg = CONFIGS["tiny_fp32"].with_(name="graph", cfg_id=13, T=T, d=d, d_ff=d_ff, dtype="bf16")
    inp = generate(cfg)
    dv = {k: to_dev(v) for k, v in inp.items()}
    shape = moe.make_shape(T, d, d_ff, 8, 2, torch.bfloat16)
    ws = torch.empty(moe.workspace_size(shape), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(dv["x"])
    args = (dv["x"], dv["w_gate"], dv["bias"], dv["w1"], dv["w3"], dv["w2"])
    eager = moe.moe_forward(*args, workspace=ws).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_forward(*args, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(*args, out=y, workspace=ws)
    for rep in range(4):
        y.zero_()
        scratch = torch.randn(1 << 16, device="cuda") * rep  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {rep} differs from eager"
        del scratch
    y_ref, (gl, _, _) = oracle.moe_forward_expert_loop(inp["x"], inp["w_gate"], None, inp["w1"], inp["w3"],
                                                       inp["w2"])
    clear, _ = clear_tokens(gl)
    assert max_rel_err(to_host(y), y_ref, clear) <= BF16_TOL
