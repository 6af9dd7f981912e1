"""GPU parity of the layer's variants beyond Mixtral's E = 8 ("Mixtral" page,
"Конфигурация", key `num_experts`; "Вопросы и упражнения", exercise 2: E = 16,
k = 2) and of the forms the other tests leave out: the residual block in fp32,
every router launch shape with and without the fused RMSNorm, and the full
prefill workload compared on every element."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_wave_amd as moe
from synth import CONFIGS, generate, generate_torch

from gpu_helpers import BF16_TOL, F32_TOL, check_routing, clear_tokens, max_rel_err, say, to_dev, to_host, widen_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()


def small(name, T, d, d_ff, E=8, k=2, dtype="bf16", cfg_id=11):
    return CONFIGS["tiny_fp32"].with_(name=name, cfg_id=cfg_id, T=T, d=d, d_ff=d_ff, E=E, k=k, dtype=dtype,
                                      x_unit_rms=False, wg_std=0.02, bias=None)


def _clear_k(g, k):
    """Tokens whose k-th and (k+1)-th logits differ by more than 1e-4 (all tokens when k == E)."""
    E = g.shape[1]
    if k == E:
        return np.ones(g.shape[0], bool)
    s = np.sort(g.astype(np.float64), axis=1)[:, ::-1]
    return (s[:, k - 1] - s[:, k]) > 1e-4


# ---------------------------------------------------------------------------
# the whole layer at E != 8, both bf16 expert paths
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,d_ff,E,k,path", [
    (16, 512, 1024, 16, 2, "stream"),   # the pages' exercise: 16 experts, top-2
    (300, 256, 384, 16, 2, "gemm"),
    (64, 512, 512, 16, 2, "stream"),
    (65, 512, 512, 16, 2, "gemm"),
    (8, 1024, 1024, 4, 2, "stream"),
    (40, 512, 1024, 2, 1, "stream"),
    (30, 512, 512, 32, 4, "stream"),
    (500, 256, 320, 64, 2, "gemm"),
    (20, 512, 512, 64, 8, "stream"),
    (200, 192, 256, 32, 3, "gemm"),
])
def test_forward_more_experts(T, d, d_ff, E, k, path):
    say(f"forward E={E} k={k} T={T} d={d} d_ff={d_ff} ({path})")
    cfg = small(f"fe{E}", T, d, d_ff, E=E, k=k)
    inp = generate(cfg)
    y_ref, (g, idx, w) = oracle.moe_forward_expert_loop(inp["x"], inp["w_gate"], None, inp["w1"], inp["w3"],
                                                        inp["w2"], k=k)
    dv = {key: to_dev(v) for key, v in inp.items()}
    y = moe.moe_forward(dv["x"], dv["w_gate"], None, dv["w1"], dv["w3"], dv["w2"], k=k)
    torch.cuda.synchronize()
    clear = _clear_k(g, k)
    assert clear.mean() > 0.8
    err = max_rel_err(to_host(y), y_ref, clear)
    say(f"  max rel err {err:.3e} on {int(clear.sum())} tokens")
    assert err <= BF16_TOL


@pytest.mark.parametrize("T,d,d_ff,E", [(16, 512, 1024, 16), (5, 1024, 512, 32), (3, 512, 1024, 64),
                                         (1000, 256, 384, 16)])
def test_expert_ffn_more_experts(T, d, d_ff, E):
    """The expert FFN alone on a fixed permutation (no routing in the loop)."""
    say(f"expert_ffn E={E} T={T} d={d} d_ff={d_ff}")
    cfg = small(f"ffe{E}", T, d, d_ff, E=E)
    inp = generate(cfg)
    g, idx, w = oracle.route_ref(inp["x"], inp["w_gate"], None)
    off, st, inv = oracle.dispatch_ref(idx, E)
    ref = oracle.expert_rows_ref(inp["x"], st, off, inp["w1"], inp["w3"], inp["w2"])
    ys = moe.moe_expert_ffn(to_dev(inp["x"]), to_dev(off), to_dev(st), to_dev(inp["w1"]), to_dev(inp["w3"]),
                            to_dev(inp["w2"]))
    torch.cuda.synchronize()
    assert max_rel_err(to_host(ys), ref) <= BF16_TOL


# ---------------------------------------------------------------------------
# router launch shapes: one token per workgroup (T <= 512) and several
# (T > 512: 2 tokens at E = 16, 1 token on four waves at E = 32 and 64)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E", [(1000, 16), (1000, 32), (777, 64), (513, 2), (2000, 4)])
def test_router_multi_token_path(T, E):
    say(f"router T={T} E={E}")
    cfg = small("rt", T, 256, 64, E=E)
    inp = generate(cfg, tensors=("x", "w_gate"))
    g_ref, idx_ref, w_ref = oracle.route_ref(inp["x"], inp["w_gate"], None)
    idx, w, logits = moe.moe_route(to_dev(inp["x"]), to_dev(inp["w_gate"]), None, want_logits=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_host(logits), g_ref, rtol=1e-5, atol=1e-5)
    check_routing(g_ref, idx_ref, w_ref, to_host(idx), to_host(w))


# ---------------------------------------------------------------------------
# the residual block (RMSNorm fused into the router) at E != 8, and in fp32
# ---------------------------------------------------------------------------
def _block_case(cfg, gamma):
    inp = generate(cfg)
    h_in = inp["x"].copy()
    dv_h = to_dev(h_in)
    moe.moe_block_forward(dv_h, to_dev(gamma), 1e-5, to_dev(inp["w_gate"]), None, to_dev(inp["w1"]),
                          to_dev(inp["w3"]), to_dev(inp["w2"]), k=cfg.k)
    torch.cuda.synchronize()
    h_out = widen_host(to_host(dv_h))
    ref, u, (g, idx, w) = oracle.block_forward_ref(h_in, gamma, 1e-5, inp["w_gate"], None, inp["w1"], inp["w3"],
                                                   inp["w2"], k=cfg.k)
    clear = _clear_k(g, cfg.k)
    assert clear.mean() > 0.8
    y_ref = ref - widen_host(h_in)
    return h_out, ref, y_ref, clear


@pytest.mark.parametrize("T,E", [(300, 16), (700, 16), (300, 32), (700, 32), (300, 64), (700, 64), (600, 4)])
def test_block_forward_more_experts(T, E):
    """Both router launch shapes (T <= 512 and above) with the fused RMSNorm; at
    E = 64 the norm's sum of squares is the 65th reduced column."""
    say(f"block E={E} T={T}")
    cfg = small(f"be{E}", T, 256, 384, E=E)
    gamma = np.linspace(0.5, 1.5, cfg.d).astype(np.float32)
    h_out, ref, y_ref, clear = _block_case(cfg, gamma)
    tol = BF16_TOL * np.max(np.abs(y_ref)) + 2 ** -8 * np.max(np.abs(ref))
    err = np.max(np.abs(h_out[clear] - ref[clear]))
    say(f"  max err {err:.3e} (tol {tol:.3e})")
    assert err <= tol


@pytest.mark.parametrize("T,E", [(333, 8), (700, 8), (200, 16)])
def test_block_forward_fp32(T, E):
    say(f"block fp32 E={E} T={T}")
    cfg = small("bf32", T, 192, 256, E=E, dtype="f32")
    gamma = np.linspace(0.75, 1.25, cfg.d).astype(np.float32)
    h_out, ref, y_ref, clear = _block_case(cfg, gamma)
    err = np.max(np.abs(h_out[clear] - ref[clear]))
    tol = F32_TOL * np.max(np.abs(y_ref))
    say(f"  max err {err:.3e} (tol {tol:.3e})")
    assert err <= tol


# ---------------------------------------------------------------------------
# the prefill workload on every element (d = 4096, d_ff = 14336, T = 4096)
# ---------------------------------------------------------------------------
def test_mixtral_prefill_t4096_every_element():
    """moe_forward as the benchmark runs it, every output element of every clear
    token against the oracle's expert-major form on the host."""
    cfg = CONFIGS["mixtral_prefill_t4096"]
    say("prefill T=4096 every element: generating")
    dv = generate_torch(cfg, torch.device("cuda:0"))
    y = moe.moe_forward(dv["x"], dv["w_gate"], None, dv["w1"], dv["w3"], dv["w2"])
    torch.cuda.synchronize()
    y = to_host(y)
    xh, wgh = to_host(dv["x"]), to_host(dv["w_gate"])
    w1, w3, w2 = to_host(dv["w1"]), to_host(dv["w3"]), to_host(dv["w2"])
    del dv
    say("prefill T=4096 every element: oracle")
    y_ref, (g, idx, w) = oracle.moe_forward_expert_loop(xh, wgh, None, w1, w3, w2)
    clear, _ = clear_tokens(g)
    err = max_rel_err(y, y_ref, clear)
    say(f"prefill T=4096 every element: max rel err {err:.3e} on {int(clear.sum())} tokens")
    assert clear.mean() > 0.95
    assert err <= BF16_TOL


def test_mixtral_skewed_t16384_every_element():
    """The Zipf-skewed workload (T = 16384, router bias ln p_e) as the benchmark
    runs it: expert loads from about 11.5k rows down to about 1k, so every
    expert ends in a ragged row tile; every output element of every clear token
    against the oracle's expert-major form on the host."""
    cfg = CONFIGS["mixtral_skewed_t16384"]
    say("skewed T=16384 every element: generating")
    dv = generate_torch(cfg, torch.device("cuda:0"))
    y = moe.moe_forward(dv["x"], dv["w_gate"], dv["bias"], dv["w1"], dv["w3"], dv["w2"])
    torch.cuda.synchronize()
    y = to_host(y)
    xh, wgh, bh = to_host(dv["x"]), to_host(dv["w_gate"]), to_host(dv["bias"])
    w1, w3, w2 = to_host(dv["w1"]), to_host(dv["w3"]), to_host(dv["w2"])
    del dv
    say("skewed T=16384 every element: oracle")
    y_ref, (g, idx, w) = oracle.moe_forward_expert_loop(xh, wgh, bh, w1, w3, w2)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    clear, _ = clear_tokens(g)
    err = max_rel_err(y, y_ref, clear)
    say(f"skewed T=16384 every element: rows per expert {counts.tolist()}, max rel err {err:.3e} "
        f"on {int(clear.sum())} tokens")
    assert counts.max() > 8 * counts.min()  # the skew is there
    assert clear.mean() > 0.95
    assert err <= BF16_TOL
