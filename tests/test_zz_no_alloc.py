"""moe_forward_noalloc, the entry point that allocates nothing (its
intermediates live in the library's static per-GPU scratch buffer), against
moe_forward on the same inputs, through the C ABI: two calls in a row, the
second with a smaller input, on the GEMM, streaming and fp32 paths."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_wave_amd as moe
from synth import CONFIGS, generate, generate_torch

from gpu_helpers import BF16_TOL, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()


def _rel(y, ref):
    y, ref = y.float(), ref.float()
    return float((y - ref).abs().max() / ref.abs().max().clamp_min(1e-30))


def _both(dv, k=2):
    args = (dv["x"], dv["w_gate"], dv["bias"], dv["w1"], dv["w3"], dv["w2"])
    ref = moe.moe_forward(*args, k=k)
    out = torch.full_like(ref, float("nan"))
    got = moe.moe_forward_noalloc(*args, k=k, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    return got, ref


def _small(name, T, d, d_ff, dtype="bf16", E=8):
    return CONFIGS["tiny_fp32"].with_(name=name, cfg_id=12, T=T, d=d, d_ff=d_ff, E=E, dtype=dtype, x_unit_rms=False,
                                      wg_std=0.02, bias=None)


@pytest.mark.parametrize("first,second", [
    # (T, d, d_ff, dtype): GEMM path, then a smaller streaming call
    ((300, 256, 384, "bf16"), (16, 512, 1024, "bf16")),
    # streaming, then smaller streaming
    ((64, 512, 512, "bf16"), (5, 512, 512, "bf16")),
    # fp32, then smaller fp32
    ((333, 192, 256, "f32"), (64, 128, 256, "f32")),
])
def test_noalloc_equals_forward_two_calls(first, second):
    for T, d, d_ff, dtype in (first, second):
        say(f"noalloc T={T} d={d} d_ff={d_ff} {dtype}")
        dv = {key: to_dev(v) for key, v in generate(_small("na", T, d, d_ff, dtype)).items()}
        got, ref = _both(dv)
        assert not torch.isnan(got.float()).any()
        if T <= 64 or dtype == "f32":
            # same kernels, same order: bit for bit
            assert torch.equal(got, ref)
        else:
            assert _rel(got, ref) <= BF16_TOL


def test_noalloc_mixtral_shape_two_calls():
    """Mixtral widths: 700 tokens on the GEMM path (just under the 744-token
    limit of the 64 MiB buffer), then the 16-token decode layer."""
    for T, name in ((700, "mixtral_prefill_t4096"), (16, "mixtral_decode_t16")):
        say(f"noalloc Mixtral T={T}")
        cfg = CONFIGS[name].with_(T=T)
        dv = generate_torch(cfg, torch.device("cuda:0"))
        got, ref = _both(dv)
        if T <= 64:
            assert torch.equal(got, ref)
        else:
            err = _rel(got, ref)
            say(f"  max rel diff {err:.3e}")
            assert err <= BF16_TOL
        again = moe.moe_forward_noalloc(dv["x"], dv["w_gate"], dv["bias"], dv["w1"], dv["w3"], dv["w2"])
        torch.cuda.synchronize()
        assert torch.equal(again, got)  # the buffer's leftovers do not leak into the next call
        del dv

