"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded
inputs.  Small shapes span several tiles with ragged tails; the Mixtral shapes
are checked in full where the oracle is quick, else on sampled tokens."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_wave_amd as moe
from synth import CONFIGS, generate, generate_torch

from gpu_helpers import (BF16_TOL, F32_TOL, check_dispatch_on_clear, check_routing, clear_tokens,
                         max_rel_err, say, to_dev, to_host, widen_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load()


def small(name, T, d, d_ff, E=8, dtype="bf16", bias=None, cfg_id=10):
    return CONFIGS["tiny_fp32"].with_(name=name, cfg_id=cfg_id, T=T, d=d, d_ff=d_ff, E=E, dtype=dtype,
                                      bias=bias, x_unit_rms=False, wg_std=0.02)


def run_forward(inp):
    dv = {k: to_dev(v) for k, v in inp.items()}
    y = moe.moe_forward(dv["x"], dv["w_gate"], dv["bias"], dv["w1"], dv["w3"], dv["w2"])
    torch.cuda.synchronize()
    return to_host(y)


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,E,dtype,bias", [
    (64, 128, 8, "f32", None),
    (300, 192, 8, "bf16", None),
    (1000, 512, 8, "bf16", "zipf1.2"),
    (37, 256, 2, "bf16", None),
    (77, 256, 4, "f32", None),
    (129, 256, 16, "bf16", None),
    (65, 256, 32, "f32", None),
    (33, 256, 64, "bf16", None),
    (1, 4096, 8, "bf16", None),
    (4097, 512, 8, "bf16", None),           # two tokens per wave group, the last ragged
    (8195, 256, 8, "bf16", "zipf1.2"),      # four tokens per wave group, the last ragged
])
def test_router_parity(T, d, E, dtype, bias):
    say(f"router T={T} d={d} E={E} {dtype} bias={bias}")
    cfg = small("router", T, d, 64, E=E, dtype=dtype, bias=("zipf1.2" if bias else None))
    inp = generate(cfg, tensors=("x", "w_gate"))
    if E != 8 and bias:
        inp["bias"] = None
    g_ref, idx_ref, w_ref = oracle.route_ref(inp["x"], inp["w_gate"], inp["bias"])
    idx, w, logits = moe.moe_route(to_dev(inp["x"]), to_dev(inp["w_gate"]), to_dev(inp["bias"]), want_logits=True)
    torch.cuda.synchronize()
    idx, w, logits = to_host(idx), to_host(w), to_host(logits)
    np.testing.assert_allclose(logits, g_ref, rtol=1e-5, atol=1e-5)
    check_routing(g_ref, idx_ref, w_ref, idx, w)


def test_router_exact_ties_go_to_lower_index():
    say("router ties")
    cfg = small("ties", 200, 256, 64)
    inp = generate(cfg, tensors=("x", "w_gate"))
    wg = inp["w_gate"].copy()
    wg[5] = wg[2]        # experts 2 and 5 always tie exactly
    wg[7] = wg[2]
    wg[2] += 0.5 * np.abs(wg[2])  # and make 2 (hence 5, 7) often win
    wg[5] = wg[2]
    wg[7] = wg[2]
    idx, w, logits = moe.moe_route(to_dev(inp["x"]), to_dev(wg), None, want_logits=True)
    torch.cuda.synchronize()
    idx, logits = to_host(idx), to_host(logits)
    assert np.array_equal(logits[:, 2], logits[:, 5]) and np.array_equal(logits[:, 2], logits[:, 7])
    # wherever expert 2 is the best logit, the pair is (2, 5): ties go to the lower index
    top = np.argmax(logits, axis=1)
    sel = top == 2
    assert sel.sum() > 10
    assert np.all(idx[sel, 0] == 2) and np.all(idx[sel, 1] == 5)
    assert not np.any(idx == 7)


# ---------------------------------------------------------------------------
# dispatch (integer work: bit-exact on identical inputs)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,mode", [
    (1, 8, "random"), (16, 8, "random"), (1000, 8, "random"), (16384, 8, "zipf"),
    (4097, 16, "random"), (500, 64, "random"), (300, 2, "random"), (2048, 8, "one_pair"),
    (700, 8, "empty_experts"),
])
def test_dispatch_bit_exact(T, E, mode):
    say(f"dispatch T={T} E={E} {mode}")
    rng = np.random.default_rng(T * 131 + E)
    g = rng.standard_normal((T, E)).astype(np.float32)
    if mode == "zipf":
        g += np.log(np.arange(1, E + 1, dtype=np.float32) ** -1.2)[None, :] * 3
    if mode == "one_pair":
        g[:, 3] += 100
        g[:, 5] += 100
    if mode == "empty_experts":
        g[:, [0, 4, 6]] -= 100
    idx = oracle.top2(g)
    off_ref, st_ref, inv_ref = oracle.dispatch_ref(idx, E)
    off, st, inv = moe.moe_dispatch(to_dev(idx), E)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(off), off_ref)
    assert np.array_equal(to_host(st), st_ref)
    assert np.array_equal(to_host(inv), inv_ref)


@pytest.mark.parametrize("T,E,k", [
    (3000, 8, 1), (700, 8, 4), (2000, 16, 3), (5000, 4, 4), (600, 8, 3),
])
def test_dispatch_bit_exact_general_k(T, E, k):
    """k distinct experts per token, drawn at random; T * k spans both sides
    of the 2048-pair switch to the one-workgroup-per-256-pairs kernel."""
    say(f"dispatch T={T} E={E} k={k}")
    rng = np.random.default_rng(T * 7 + E * 3 + k)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    off_ref, st_ref, inv_ref = oracle.dispatch_ref(idx, E)
    off, st, inv = moe.moe_dispatch(to_dev(idx), E)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(off), off_ref)
    assert np.array_equal(to_host(st), st_ref)
    assert np.array_equal(to_host(inv), inv_ref)


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,out_dtype,residual", [
    (100, 256, torch.float32, False), (300, 192, torch.bfloat16, False), (257, 4096, torch.bfloat16, True),
    (64, 128, torch.float32, True),
])
def test_combine(T, d, out_dtype, residual):
    say(f"combine T={T} d={d} {out_dtype} residual={residual}")
    rng = np.random.default_rng(T + d)
    idx = oracle.top2(rng.standard_normal((T, 8)).astype(np.float32))
    off, st, inv = oracle.dispatch_ref(idx, 8)
    ys = rng.standard_normal((2 * T, d)).astype(np.float32)
    w = rng.uniform(0, 1, (T, 2)).astype(np.float32)
    res = None
    if residual:
        res = rng.standard_normal((T, d)).astype(np.float32)
        if out_dtype == torch.bfloat16:
            from synth import bf16_bits_from_f32
            res = bf16_bits_from_f32(res)
    ref = oracle.combine_ref(ys, inv, w, res)
    y = moe.moe_combine(to_dev(ys), to_dev(inv), to_dev(w), 8, out_dtype=out_dtype, residual=to_dev(res))
    torch.cuda.synchronize()
    y = widen_host(to_host(y))
    if out_dtype == torch.bfloat16:
        assert np.all(np.abs(y - ref) <= np.abs(ref) * 2 ** -8 + 1e-6)
    else:
        np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)


def test_combine_residual_may_alias_output():
    say("combine aliased residual")
    T, d = 50, 256
    rng = np.random.default_rng(1)
    idx = oracle.top2(rng.standard_normal((T, 8)).astype(np.float32))
    _, _, inv = oracle.dispatch_ref(idx, 8)
    ys = rng.standard_normal((2 * T, d)).astype(np.float32)
    w = rng.uniform(0, 1, (T, 2)).astype(np.float32)
    h = rng.standard_normal((T, d)).astype(np.float32)
    ref = oracle.combine_ref(ys, inv, w, h)
    hd = to_dev(h)
    moe.moe_combine(to_dev(ys), to_dev(inv), to_dev(w), 8, out_dtype=torch.float32, residual=hd, out=hd)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_host(hd), ref, rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------------------
# expert FFN (both bf16 paths and fp32)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,d_ff,dtype,path", [
    (64, 128, 256, "f32", "gemm"),
    (300, 192, 320, "bf16", "gemm"),
    (1000, 256, 384, "bf16", "gemm"),
    (5, 512, 1024, "bf16", "stream"),
    (3, 1024, 1024, "bf16", "stream"),
    (8, 1024, 2048, "bf16", "stream"),    # 16-column items, 8-way K split, up and down
    (6, 2048, 1024, "bf16", "stream"),
    (2, 512, 1024, "bf16", "stream"),
    (16, 512, 1536, "bf16", "stream"),
    (30, 1024, 512, "bf16", "stream"),
    (64, 512, 1024, "bf16", "stream"),
    (65, 512, 1024, "bf16", "gemm"),  # one token past the streaming limit, same widths
    (16, 192, 256, "bf16", "gemm"),   # d not a multiple of 512: small T on the GEMM path
    (100, 64, 64, "bf16", "gemm"),    # K = 64: two 32-wide slices, the shortest main loop
    (200, 128, 128, "bf16", "gemm"),  # four slices: no ten-slice trip, two tail pairs
    (130, 64, 832, "bf16", "gemm"),   # up: 2 slices; down: 26 = 20 + 6; d_ff not a multiple of 128
])
def test_expert_ffn(T, d, d_ff, dtype, path):
    say(f"expert_ffn T={T} d={d} d_ff={d_ff} {dtype} {path}")
    cfg = small("ffn", T, d, d_ff, dtype=dtype)
    inp = generate(cfg)
    g, idx, w = oracle.route_ref(inp["x"], inp["w_gate"], None)
    off, st, inv = oracle.dispatch_ref(idx, 8)
    ref = oracle.expert_rows_ref(inp["x"], st, off, inp["w1"], inp["w3"], inp["w2"])
    ys = moe.moe_expert_ffn(to_dev(inp["x"]), to_dev(off), to_dev(st), to_dev(inp["w1"]), to_dev(inp["w3"]),
                            to_dev(inp["w2"]))
    torch.cuda.synchronize()
    err = max_rel_err(to_host(ys), ref)
    assert err <= (F32_TOL if dtype == "f32" else BF16_TOL), err


@pytest.mark.parametrize("d,d_ff,counts", [
    (512, 1024, [1024, 1024]),         # up 64 tiles in 4 K pieces, down 16 tiles in 8
    (1024, 2048, [300, 257, 1, 700]),  # ragged experts: up 128 tiles in 2 pieces, down 32 tiles in 8
    (512, 4096, [1500, 1100]),         # up 352 tiles: 256 whole, 96 in 2 pieces; down 22 tiles in 8
    (512, 1024, [1024, 0]),            # one expert-parallel rank: every row on one local expert
])
def test_expert_ffn_split_last_round(d, d_ff, counts):
    """The grouped GEMM splits the tiles of its last round along K (on a
    256-CU part: the piece counts noted above) and sums the pieces in a
    fix-up pass; rows are routed by hand so the tile counts are known."""
    E, T = len(counts), sum(counts)
    say(f"expert_ffn split d={d} d_ff={d_ff} counts={counts}")
    inp = generate(small("split", T, d, d_ff, E=E))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    st = np.random.default_rng(T).permutation(T).astype(np.int32)
    ref = oracle.expert_rows_ref(inp["x"], st, off, inp["w1"], inp["w3"], inp["w2"])
    args = (to_dev(inp["x"]), to_dev(off), to_dev(st), to_dev(inp["w1"]), to_dev(inp["w3"]), to_dev(inp["w2"]))
    ys = moe.moe_expert_ffn(*args, k=1).clone()
    again = moe.moe_expert_ffn(*args, k=1)
    torch.cuda.synchronize()
    assert max_rel_err(to_host(ys), ref) <= BF16_TOL
    assert torch.equal(ys, again)  # the pieces are summed in a fixed order


def test_expert_ffn_tile_row_boundaries():
    """Every partial-tile case of the grouped GEMM in one call: experts whose
    last 256-row tile holds 1, 15 .. 17, 31 .. 33, 127 .. 129 rows (16-row
    blocks skipped), 223 .. 225 rows (the switch to the branch-free main loop
    above 224) and 255 .. 257 rows, the rows gathered in a random order; rows
    routed by hand, every row against the oracle."""
    counts = [1, 15, 16, 17, 31, 32, 33, 127, 128, 129, 223, 224, 225, 255, 256, 257]
    E, T, d, d_ff = len(counts), sum(counts), 256, 512
    say(f"expert_ffn tile-row boundaries E={E} T={T}")
    inp = generate(small("rowbound", T, d, d_ff, E=E))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    st = np.random.default_rng(11).permutation(T).astype(np.int32)
    ref = oracle.expert_rows_ref(inp["x"], st, off, inp["w1"], inp["w3"], inp["w2"])
    ys = moe.moe_expert_ffn(to_dev(inp["x"]), to_dev(off), to_dev(st), to_dev(inp["w1"]), to_dev(inp["w3"]),
                            to_dev(inp["w2"]), k=1)
    torch.cuda.synchronize()
    assert max_rel_err(to_host(ys), ref) <= BF16_TOL


# ---------------------------------------------------------------------------
# the whole layer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [
    CONFIGS["tiny_fp32"],
    small("small_bf16", 1000, 256, 384),
    small("small_bf16_ragged", 300, 192, 320, bias="zipf1.2"),
    small("small_decode", 16, 512, 1024),
    small("small_decode40", 40, 512, 1024),
    small("t1", 1, 256, 512),
    small("t1_stream", 1, 512, 512),
    small("small_fp32", 333, 192, 256, dtype="f32"),
], ids=lambda c: c.name)
def test_forward_small(cfg):
    say(f"forward {cfg.name} T={cfg.T} d={cfg.d} d_ff={cfg.d_ff} {cfg.dtype}")
    inp = generate(cfg)
    y_ref, (g, idx, w) = oracle.moe_forward_expert_loop(inp["x"], inp["w_gate"], inp["bias"], inp["w1"],
                                                        inp["w3"], inp["w2"])
    y = run_forward(inp)
    clear, _ = clear_tokens(g)
    err = max_rel_err(y, y_ref, clear)
    assert err <= (F32_TOL if cfg.dtype == "f32" else BF16_TOL), err


def test_forward_all_tokens_one_pair():
    say("forward one pair")
    cfg = small("one_pair", 500, 256, 384)
    inp = generate(cfg)
    inp["bias"] = np.zeros(8, np.float32)
    inp["bias"][[3, 5]] = 50.0
    y_ref, (g, idx, w) = oracle.moe_forward_expert_loop(inp["x"], inp["w_gate"], inp["bias"], inp["w1"],
                                                        inp["w3"], inp["w2"])
    assert np.all(np.sort(idx, axis=1) == [3, 5])
    y = run_forward(inp)
    assert max_rel_err(y, y_ref) <= BF16_TOL


def test_forward_identity_when_experts_equal():
    # All experts equal: the layer is one dense SwiGLU whatever the routing,
    # so near-tie tokens are checked too.
    say("forward identity")
    cfg = small("identity", 400, 256, 384)
    inp = generate(cfg)
    for key in ("w1", "w3", "w2"):
        inp[key] = np.ascontiguousarray(np.broadcast_to(inp[key][0], inp[key].shape))
    dense = oracle.expert_swiglu(inp["x"], inp["w1"][0], inp["w3"][0], inp["w2"][0])
    y = run_forward(inp)
    assert max_rel_err(y, dense) <= BF16_TOL


def test_forward_zero_tokens():
    say("forward T=0")
    cfg = small("t0", 4, 256, 512)
    inp = generate(cfg)
    inp["x"] = inp["x"][:0]
    dv = {k: to_dev(v) for k, v in inp.items()}
    y = moe.moe_forward(dv["x"], dv["w_gate"], None, dv["w1"], dv["w3"], dv["w2"])
    torch.cuda.synchronize()
    assert y.shape == (0, 256)


def test_forward_is_deterministic():
    say("forward determinism")
    cfg = small("det", 777, 256, 384)
    inp = generate(cfg)
    a, b = run_forward(inp), run_forward(inp)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("T", [300, 701])
def test_block_forward_two_layers_teacher_forced(T):
    """T = 300 routes one token per workgroup, T = 701 four (the last one
    ragged), both with the RMSNorm fused into the router."""
    cfg = small("block", T, 256, 384)
    dv_h = None
    for layer in range(2):
        say(f"block T={T} layer {layer}")
        inp = generate(cfg, layer=layer)
        if dv_h is None:
            dv_h = to_dev(inp["x"])
        h_in = to_host(dv_h).copy()
        gamma = np.linspace(0.5, 1.5, cfg.d).astype(np.float32)
        moe.moe_block_forward(dv_h, to_dev(gamma), 1e-5, to_dev(inp["w_gate"]), None, to_dev(inp["w1"]),
                              to_dev(inp["w3"]), to_dev(inp["w2"]))
        torch.cuda.synchronize()
        h_out = widen_host(to_host(dv_h))
        ref, u, (g, idx, w) = oracle.block_forward_ref(h_in, gamma, 1e-5, inp["w_gate"], None, inp["w1"],
                                                       inp["w3"], inp["w2"])
        y_ref = ref - widen_host(h_in)
        clear, _ = clear_tokens(g)
        tol = BF16_TOL * np.max(np.abs(y_ref)) + 2 ** -8 * np.max(np.abs(ref))
        assert np.max(np.abs(h_out[clear] - ref[clear])) <= tol


# ---------------------------------------------------------------------------
# Mixtral shapes
# ---------------------------------------------------------------------------
def _mixtral_case(name, sample):
    cfg = CONFIGS[name] if isinstance(name, str) else name
    name = cfg.name
    say(f"mixtral {name}: generating")
    dv = generate_torch(cfg, torch.device("cuda:0"))
    x, wg, b = dv["x"], dv["w_gate"], dv["bias"]
    say(f"mixtral {name}: route + dispatch + forward")
    idx, w, _ = moe.moe_route(x, wg, b)
    off, st, inv = moe.moe_dispatch(idx, cfg.E)
    y = moe.moe_forward(x, wg, b, dv["w1"], dv["w3"], dv["w2"])
    torch.cuda.synchronize()
    say(f"mixtral {name}: oracle")
    xh, wgh = to_host(x), to_host(wg)
    bh = to_host(b) if b is not None else None
    g_ref, idx_ref, w_ref = oracle.route_ref(xh, wgh, bh)
    idx_h = to_host(idx)
    clear = check_routing(g_ref, idx_ref, w_ref, idx_h, to_host(w))
    check_dispatch_on_clear(idx_h, to_host(off), to_host(st), to_host(inv), clear, cfg.E)
    # per expert, GPU rows minus near-tie tokens == oracle rows minus near-tie tokens
    off_ref, st_ref, _ = oracle.dispatch_ref(idx_ref, cfg.E)
    off_h, st_h = to_host(off), to_host(st)
    for e in range(cfg.E):
        a = [t for t in st_h[off_h[e]:off_h[e + 1]] if clear[t]]
        r = [t for t in st_ref[off_ref[e]:off_ref[e + 1]] if clear[t]]
        assert a == r, f"expert {e} rows differ"
    counts = np.diff(off_h)
    say(f"mixtral {name}: rows per expert {counts.tolist()}")
    tokens = sample(cfg, counts, idx_h, clear)
    w1, w3, w2 = to_host(dv["w1"]), to_host(dv["w3"]), to_host(dv["w2"])
    y_ref, _ = oracle.moe_forward_tokens(xh[tokens], wgh, bh, w1, w3, w2)
    err = max_rel_err(to_host(y)[tokens], y_ref)
    say(f"mixtral {name}: max rel err {err:.3e} on {len(tokens)} tokens")
    assert err <= BF16_TOL


def _sample_tokens(cfg, counts, idx, clear, n=24):
    rng = np.random.default_rng(7)
    T = cfg.T
    picks = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    picks.update([0, T - 1])
    # tokens of the lightest and heaviest experts
    for e in (int(np.argmin(counts)), int(np.argmax(counts))):
        picks.update(np.nonzero(np.any(idx == e, axis=1))[0][-3:].tolist())
    return np.array(sorted(t for t in picks if clear[t]), dtype=np.int64)


def test_mixtral_decode_t16_full():
    _mixtral_case("mixtral_decode_t16", lambda cfg, c, i, cl: np.nonzero(cl)[0])


@pytest.mark.parametrize("T", [1, 2, 4, 8])
def test_mixtral_decode_small_t_full(T):
    """The small-T decode layers of the latency sweep (Mixtral decode weights,
    T = 1 .. 8 tokens, the 16-column / 8-way-K-split streaming shapes): every
    token against the oracle."""
    cfg = CONFIGS["mixtral_decode_t16"].with_(name=f"mixtral_decode_t{T}", T=T)
    _mixtral_case(cfg, lambda cfg, c, i, cl: np.nonzero(cl)[0])


def test_ep_rank_share_sampled():
    """One expert-parallel rank's share as bench.py times it: 1024 rows through
    one local expert at full width (d = 4096, d_ff = 14336; a second, empty
    expert in the layout), on the grouped GEMM.  Sampled rows against the
    oracle, which computes just those rows."""
    rows = 1024
    cfg = CONFIGS["mixtral_prefill_t4096"].with_(name="ep_rank_t4096", T=rows, E=2, k=1)
    say("ep rank share: generating")
    dv = generate_torch(cfg, torch.device("cuda:0"))
    dev = dv["x"].device
    off = torch.tensor([0, rows, rows], dtype=torch.int32, device=dev)
    st = torch.arange(rows, dtype=torch.int32, device=dev)
    ys = moe.moe_expert_ffn(dv["x"], off, st, dv["w1"], dv["w3"], dv["w2"], k=1)
    torch.cuda.synchronize()
    picks = np.array(sorted({0, 1, 255, 256, 511, 767, 1023, *np.random.default_rng(3).integers(0, rows, 9).tolist()}),
                     dtype=np.int32)
    say(f"ep rank share: oracle on {len(picks)} rows")
    off_s = np.array([0, len(picks), len(picks)], dtype=np.int32)
    ref = oracle.expert_rows_ref(to_host(dv["x"]), picks, off_s, to_host(dv["w1"]), to_host(dv["w3"]),
                                 to_host(dv["w2"]))
    assert max_rel_err(to_host(ys)[picks], ref) <= BF16_TOL


def test_mixtral_prefill_t4096_sampled():
    _mixtral_case("mixtral_prefill_t4096", _sample_tokens)


def test_mixtral_skewed_t16384_sampled():
    _mixtral_case("mixtral_skewed_t16384", _sample_tokens)


def test_mixtral_prefill_t65536_sampled():
    """The largest size tested: 131072 dispatched rows, a grid of ~58k GEMM
    workgroups; every token's routing and the permutation are checked, outputs
    on sampled tokens."""
    cfg = CONFIGS["mixtral_prefill_t4096"].with_(name="mixtral_prefill_t65536", cfg_id=30, T=65536)
    _mixtral_case(cfg, _sample_tokens)


def test_mixtral_stack_layers_teacher_forced():
    """Two pre-RMSNorm residual MoE sublayers at Mixtral shape (T = 2048), each
    checked on sampled tokens against the oracle fed the GPU's exact input."""
    cfg = CONFIGS["mixtral_stack32_t2048"]
    dev = torch.device("cuda:0")
    gamma = torch.ones(cfg.d, dtype=torch.float32, device=dev)
    h = None
    for layer in range(2):
        say(f"stack layer {layer}: generating")
        lw = generate_torch(cfg, dev, layer=layer)
        if h is None:
            h = lw["x"].clone()
        h_in = to_host(h).copy()
        say(f"stack layer {layer}: block forward")
        moe.moe_block_forward(h, gamma, 1e-5, lw["w_gate"], None, lw["w1"], lw["w3"], lw["w2"])
        torch.cuda.synchronize()
        h_out = widen_host(to_host(h))
        rng = np.random.default_rng(layer)
        tokens = np.sort(rng.choice(cfg.T, size=16, replace=False))
        w1, w3, w2 = to_host(lw["w1"]), to_host(lw["w3"]), to_host(lw["w2"])
        ref, u, (g, idx, w) = oracle.block_forward_ref(h_in[tokens], np.ones(cfg.d, np.float32), 1e-5,
                                                       to_host(lw["w_gate"]), None, w1, w3, w2)
        clear, _ = clear_tokens(g)
        y_ref = ref - widen_host(h_in[tokens])
        tol = BF16_TOL * np.max(np.abs(y_ref)) + 2 ** -8 * np.max(np.abs(ref))
        err = np.max(np.abs(h_out[tokens][clear] - ref[clear]))
        say(f"stack layer {layer}: max err {err:.3e} (tol {tol:.3e}) on {int(clear.sum())} tokens")
        assert err <= tol
        del lw, w1, w3, w2


# ---------------------------------------------------------------------------
# general top-k (the pages' top_k_experts parameter; Mixtral uses 2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,d,E,k", [(300, 256, 8, 1), (300, 256, 8, 3), (129, 512, 16, 4), (64, 256, 8, 8),
                                      (77, 256, 64, 6)])
def test_router_general_k(T, d, E, k):
    say(f"router general k: T={T} d={d} E={E} k={k}")
    cfg = small("rk", T, d, 64, E=E)
    inp = generate(cfg, tensors=("x", "w_gate"))
    g_ref, idx_ref, w_ref = oracle.route_ref(inp["x"], inp["w_gate"], None, k=k)
    idx, w, _ = moe.moe_route(to_dev(inp["x"]), to_dev(inp["w_gate"]), None, k=k)
    torch.cuda.synchronize()
    idx, w = to_host(idx), to_host(w)
    s = np.sort(g_ref.astype(np.float64), axis=1)[:, ::-1]
    gaps = np.diff(-s, axis=1)  # s_j - s_{j+1} >= 0
    ok = np.all(gaps[:, :k] > 1e-4, axis=1) if k < E else np.all(gaps[:, :k - 1] > 1e-4, axis=1)
    assert ok.mean() > 0.8
    assert np.array_equal(idx[ok], idx_ref[ok])  # clear tokens: same experts in the same order
    np.testing.assert_allclose(w[ok], w_ref[ok], atol=1e-6)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert all(len(set(r)) == k for r in idx.tolist())


@pytest.mark.parametrize("T,d,d_ff,k", [(500, 256, 384, 1), (300, 192, 320, 3), (16, 512, 1024, 4),
                                         (40, 512, 512, 3), (200, 256, 256, 8)])
def test_forward_general_k(T, d, d_ff, k):
    say(f"forward general k: T={T} d={d} d_ff={d_ff} k={k}")
    cfg = small("fk", T, d, d_ff).with_(k=k)
    inp = generate(cfg)
    y_ref, (g, idx, w) = oracle.moe_forward_expert_loop(inp["x"], inp["w_gate"], None, inp["w1"], inp["w3"],
                                                        inp["w2"], k=k)
    dv = {key: to_dev(v) for key, v in inp.items()}
    y = to_host(moe.moe_forward(dv["x"], dv["w_gate"], None, dv["w1"], dv["w3"], dv["w2"], k=k))
    torch.cuda.synchronize()
    s = np.sort(g.astype(np.float64), axis=1)[:, ::-1]
    gaps = np.diff(-s, axis=1)
    clear = np.all(gaps[:, :k] > 1e-4, axis=1) if k < 8 else np.ones(T, bool)
    assert max_rel_err(y, y_ref, clear) <= BF16_TOL


# ---------------------------------------------------------------------------
# expert Linear biases ("Mixtral" page, "Конфигурация", key `bias`)
# ---------------------------------------------------------------------------
def _eb(inp, which="b1b3b2"):
    return tuple(inp[n] if n in which else None for n in ("b1", "b3", "b2"))


def _eb_dev(eb):
    return dict(zip(("b1", "b3", "b2"), (to_dev(b) for b in eb)))


@pytest.mark.parametrize("T,d,d_ff,dtype,path,which", [
    (64, 128, 256, "f32", "gemm", "b1b3b2"),
    (300, 192, 320, "bf16", "gemm", "b1b3b2"),
    (1000, 256, 384, "bf16", "gemm", "b3"),
    (16, 512, 1024, "bf16", "stream", "b1b3b2"),
    (3, 1024, 1024, "bf16", "stream", "b1b3b2"),
    (40, 512, 512, "bf16", "stream", "b2"),
])
def test_expert_ffn_with_biases(T, d, d_ff, dtype, path, which):
    say(f"expert_ffn biases T={T} d={d} d_ff={d_ff} {dtype} {path} {which}")
    cfg = small("ffnb", T, d, d_ff, dtype=dtype).with_(expert_bias_std=0.1)
    inp = generate(cfg)
    g, idx, w = oracle.route_ref(inp["x"], inp["w_gate"], None)
    off, st, inv = oracle.dispatch_ref(idx, 8)
    eb = _eb(inp, which)
    ref = oracle.expert_rows_ref(inp["x"], st, off, inp["w1"], inp["w3"], inp["w2"], eb=eb)
    ys = moe.moe_expert_ffn(to_dev(inp["x"]), to_dev(off), to_dev(st), to_dev(inp["w1"]), to_dev(inp["w3"]),
                            to_dev(inp["w2"]), **_eb_dev(eb))
    torch.cuda.synchronize()
    err = max_rel_err(to_host(ys), ref)
    assert err <= (F32_TOL if dtype == "f32" else BF16_TOL), err


@pytest.mark.parametrize("cfg", [
    small("fwd_bias_bf16", 1000, 256, 384),
    small("fwd_bias_decode", 16, 512, 1024),
    small("fwd_bias_t1", 1, 512, 512),
    small("fwd_bias_fp32", 333, 192, 256, dtype="f32"),
], ids=lambda c: c.name)
def test_forward_with_expert_biases(cfg):
    say(f"forward biases {cfg.name}")
    cfg = cfg.with_(expert_bias_std=0.1)
    inp = generate(cfg)
    eb = _eb(inp)
    y_ref, (g, idx, w) = oracle.moe_forward_expert_loop(inp["x"], inp["w_gate"], None, inp["w1"], inp["w3"],
                                                        inp["w2"], eb=eb)
    dv = {key: to_dev(v) for key, v in inp.items()}
    y = moe.moe_forward(dv["x"], dv["w_gate"], None, dv["w1"], dv["w3"], dv["w2"], **_eb_dev(eb))
    torch.cuda.synchronize()
    clear, _ = clear_tokens(g)
    assert max_rel_err(to_host(y), y_ref, clear) <= (F32_TOL if cfg.dtype == "f32" else BF16_TOL)


def test_zero_expert_biases_equal_none():
    say("forward zero biases == none")
    cfg = small("fwd_zero_bias", 300, 256, 384)
    inp = generate(cfg)
    dv = {key: to_dev(v) for key, v in inp.items()}
    z = lambda n: torch.zeros((8, n), dtype=torch.bfloat16, device=dv["x"].device)
    y0 = moe.moe_forward(dv["x"], dv["w_gate"], None, dv["w1"], dv["w3"], dv["w2"])
    y1 = moe.moe_forward(dv["x"], dv["w_gate"], None, dv["w1"], dv["w3"], dv["w2"], b1=z(384), b3=z(384),
                         b2=z(256))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_block_forward_with_expert_biases():
    say("block forward biases")
    cfg = small("blockb", 300, 256, 384).with_(expert_bias_std=0.1)
    inp = generate(cfg)
    eb = _eb(inp)
    h_in = inp["x"].copy()
    dv_h = to_dev(h_in)
    gamma = np.ones(cfg.d, np.float32)
    moe.moe_block_forward(dv_h, to_dev(gamma), 1e-5, to_dev(inp["w_gate"]), None, to_dev(inp["w1"]),
                          to_dev(inp["w3"]), to_dev(inp["w2"]), **_eb_dev(eb))
    torch.cuda.synchronize()
    h_out = widen_host(to_host(dv_h))
    ref, u, (g, idx, w) = oracle.block_forward_ref(h_in, gamma, 1e-5, inp["w_gate"], None, inp["w1"], inp["w3"],
                                                   inp["w2"], eb=eb)
    y_ref = ref - widen_host(h_in)
    clear, _ = clear_tokens(g)
    tol = BF16_TOL * np.max(np.abs(y_ref)) + 2 ** -8 * np.max(np.abs(ref))
    assert np.max(np.abs(h_out[clear] - ref[clear])) <= tol
