"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: numbers the
pages print, closed forms, invariants, brute force on tiny inputs, or an
independent library formulation (torch / scipy / math.fsum).  The last block
plants mistakes into copies of oracle functions (on the CPU) and checks that
the pins catch them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import moe_ref
from oracle.params import mistral_param_count, moe_model_param_counts
from synth import CONFIGS, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "param_counts.txt")


# ---------------------------------------------------------------------------
# parameter counts (the pages' exact integers)
# ---------------------------------------------------------------------------
def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            model, part, value = line.split()
            out[(model, part)] = int(value)
    return out


def test_param_counts_match_pages():
    g = _golden()
    mix = moe_model_param_counts(4096, 32, 32, 8, 128, 14336, 8, 2, 32000)
    teach = moe_model_param_counts(256, 4, 4, 2, 64, 1024, 8, 2, 1000, bias=True)
    e16 = moe_model_param_counts(4096, 32, 32, 8, 128, 14336, 16, 2, 32000)
    got = {("mixtral", p): v for p, v in mix.items()}
    got.update({("teach", p): v for p, v in teach.items()})
    got.update({("e16", p): v for p, v in e16.items()})
    got[("mistral", "total")] = mistral_param_count(4096, 32, 32, 8, 128, 14336, 32000)
    got[("mistral_mha", "total")] = mistral_param_count(4096, 32, 32, 32, 128, 14336, 32000)
    got[("mistral_teach", "total")] = mistral_param_count(256, 4, 4, 2, 64, 1024, 1000, bias=True)
    assert len(g) >= 20
    for key, value in g.items():
        assert got[key] == value, key


def test_ffn_share_of_layer_flops():
    # "Mixtral" page, exercise 3: FFN share ~ 0.894 of a layer's non-quadratic FLOPs.
    c = moe_model_param_counts(4096, 32, 32, 8, 128, 14336, 8, 2, 32000)
    share = 2 * c["expert"] / (c["attention_layer"] + c["router_layer"] + 2 * c["expert"])
    assert abs(share - 0.894) < 5e-4


def test_expert_work_is_k_over_E():
    # "Алгоритм": experts process kN rows, k/E = 1/4 of all-experts-on-all-tokens.
    rng = np.random.default_rng(3)
    g = rng.standard_normal((500, 8)).astype(np.float32)
    idx = oracle.top2(g)
    off, _, _ = oracle.dispatch_ref(idx, 8)
    assert off[-1] == 2 * 500
    assert off[-1] / (8 * 500) == 0.25


# ---------------------------------------------------------------------------
# router logits: fp32 within the dot-product error bound of the exact value
# ---------------------------------------------------------------------------
def test_router_logits_within_dot_product_bound():
    cfg = CONFIGS["tiny_fp32"]
    inp = generate(cfg)
    x, wg = inp["x"], inp["w_gate"]
    g = oracle.router_logits(x, wg)
    d = x.shape[1]
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    for t in range(0, x.shape[0], 7):
        for e in range(wg.shape[0]):
            prods = [float(a) * float(b) for a, b in zip(x[t], wg[e])]  # exact in fp64
            exact = math.fsum(prods)
            bound = gamma * math.fsum(abs(p) for p in prods)
            assert abs(float(g[t, e]) - exact) <= bound + 1e-30


def test_router_bias_is_added_per_expert():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 16)).astype(np.float32)
    wg = rng.standard_normal((4, 16)).astype(np.float32)
    b = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    diff = oracle.router_logits(x, wg, b) - oracle.router_logits(x, wg)
    np.testing.assert_allclose(diff, np.broadcast_to(b, diff.shape), atol=1e-5)


# ---------------------------------------------------------------------------
# top-2: brute force over the 28 expert pairs, ties, distinctness
# ---------------------------------------------------------------------------
def _pair_argmax(gt):
    E = len(gt)
    return max(itertools.combinations(range(E), 2), key=lambda p: (gt[p[0]] + gt[p[1]]))


def test_28_pairs():
    assert len(list(itertools.combinations(range(8), 2))) == 28 == math.comb(8, 2)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_top2_set_equals_best_pair(seed):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((400, 8)).astype(np.float32)
    idx = oracle.top2(g)
    for t in range(g.shape[0]):
        srt = np.sort(g[t])[::-1]
        if srt[1] == srt[2]:
            continue
        assert set(idx[t].tolist()) == set(_pair_argmax(g[t].astype(np.float64)))
        assert idx[t, 0] != idx[t, 1]
        assert g[t, idx[t, 0]] >= g[t, idx[t, 1]]


def test_top2_tie_rule():
    g = np.array([[1, 3, 3, 0, 0, 0, 0, 0],
                  [5, 5, 5, 5, 5, 5, 5, 5],
                  [0, 0, 0, 0, 0, 0, 2, 2],
                  [0, 9, 0, 0, 0, 0, 0, 1]], np.float32)
    idx = oracle.top2(g)
    assert idx.tolist() == [[1, 2], [0, 1], [6, 7], [1, 7]]


# ---------------------------------------------------------------------------
# combine weights: sum to one, closed form, the HF softmax-then-renormalise form
# ---------------------------------------------------------------------------
def test_weights_sum_to_one_and_match_sigmoid_and_hf_form():
    rng = np.random.default_rng(5)
    g = (rng.standard_normal((1000, 8)) * 3).astype(np.float32)
    idx = oracle.top2(g)
    w = oracle.topk_softmax(g, idx)
    assert w.dtype == np.float32
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=2 ** -23 * 2)
    sel = np.take_along_axis(g.astype(np.float64), idx, axis=1)
    # closed form: w0 = sigmoid(g_s0 - g_s1)
    np.testing.assert_allclose(w[:, 0], scipy.special.expit(sel[:, 0] - sel[:, 1]), atol=1e-6)
    # HF form: softmax over all E, keep top-2, renormalise (the pages state equality)
    full = scipy.special.softmax(g.astype(np.float64), axis=1)
    keep = np.take_along_axis(full, idx, axis=1)
    np.testing.assert_allclose(w, keep / keep.sum(axis=1, keepdims=True), atol=1e-6)


def test_weights_are_zero_outside_selected_pair_via_minus_inf():
    # Top2 sets non-selected logits to -inf; a softmax over the full vector
    # then gives the same two weights and exact zeros elsewhere.
    rng = np.random.default_rng(6)
    g = rng.standard_normal((50, 8)).astype(np.float64)
    idx = oracle.top2(g)
    w = oracle.topk_softmax(g, idx, dtype=np.float64)
    masked = np.full_like(g, -np.inf)
    np.put_along_axis(masked, idx, np.take_along_axis(g, idx, axis=1), axis=1)
    sm = scipy.special.softmax(masked, axis=1)
    for t in range(g.shape[0]):
        assert np.count_nonzero(sm[t]) == 2
        np.testing.assert_allclose(sm[t, idx[t]], w[t], rtol=1e-12)


# ---------------------------------------------------------------------------
# dispatch: invariants and a nested-loop brute force
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E", [(1, 8), (37, 8), (256, 8), (100, 4)])
def test_dispatch_invariants_and_bruteforce(T, E):
    rng = np.random.default_rng(T)
    g = rng.standard_normal((T, E)).astype(np.float32)
    g[:, 2 % E] -= 50.0  # one expert never selected
    idx = oracle.top2(g)
    off, st, inv = oracle.dispatch_ref(idx, E)
    assert off[0] == 0 and off[-1] == 2 * T
    assert np.all(np.diff(off) >= 0)
    assert off[(2 % E) + 1] - off[2 % E] == 0
    counts = np.bincount(st, minlength=T)
    assert np.all(counts == 2)
    for e in range(E):
        rows = st[off[e]:off[e + 1]]
        assert np.all(np.diff(rows) > 0)
    # brute force: walk experts, then tokens, then slots
    expect = []
    for e in range(E):
        for t in range(T):
            for s in range(2):
                if idx[t, s] == e:
                    expect.append((t, s))
    assert st.tolist() == [t for t, _ in expect]
    for r, (t, s) in enumerate(expect):
        assert inv[t, s] == r


# ---------------------------------------------------------------------------
# layer output: identity case, 28-pair brute force, O1 vs O2, fp64 shadow
# ---------------------------------------------------------------------------
def _torch_swiglu(u, w1, w3, w2):
    return (torch.nn.functional.silu(u @ w1.T) * (u @ w3.T)) @ w2.T


def _tiny(seed, T=12, d=16, d_ff=24, E=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = rng.standard_normal((E, d)).astype(np.float32)
    w1 = (rng.standard_normal((E, d_ff, d)) / math.sqrt(d)).astype(np.float32)
    w3 = (rng.standard_normal((E, d_ff, d)) / math.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((E, d, d_ff)) / math.sqrt(d_ff)).astype(np.float32)
    return x, wg, w1, w3, w2


def test_identity_when_all_experts_equal():
    cfg = CONFIGS["tiny_fp32"]
    inp = generate(cfg)
    w1 = np.broadcast_to(inp["w1"][3], inp["w1"].shape).copy()
    w3 = np.broadcast_to(inp["w3"][3], inp["w3"].shape).copy()
    w2 = np.broadcast_to(inp["w2"][3], inp["w2"].shape).copy()
    y, _ = oracle.moe_forward_expert_loop(inp["x"], inp["w_gate"], None, w1, w3, w2)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    dense = _torch_swiglu(t(inp["x"]), t(w1[0]), t(w3[0]), t(w2[0])).numpy()
    assert np.max(np.abs(y - dense)) <= 1e-5 * np.max(np.abs(dense))


def _pair_bruteforce_torch(x, wg, b, w1, w3, w2):
    """y_t from the best of the 28 pairs, computed with torch in float64."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    X, WG = t(x), t(wg)
    G = X @ WG.T + (t(b) if b is not None else 0)
    T, E = G.shape
    y = torch.zeros_like(X)
    ok = np.ones(T, bool)
    for tt in range(T):
        gt = G[tt]
        srt = torch.sort(gt, descending=True).values
        ok[tt] = bool(srt[1] - srt[2] > 1e-3)
        i, j = _pair_argmax(gt.tolist())
        wts = torch.softmax(torch.stack([gt[i], gt[j]]), dim=0)
        for wgt, e in zip(wts, (i, j)):
            y[tt] += wgt * _torch_swiglu(X[tt:tt + 1], t(w1[e]), t(w3[e]), t(w2[e]))[0]
    return y.numpy(), ok


@pytest.mark.parametrize("seed", [0, 1])
def test_output_equals_28_pair_bruteforce(seed):
    x, wg, w1, w3, w2 = _tiny(seed)
    b = np.linspace(-0.5, 0.5, 8).astype(np.float32)
    y, _ = oracle.moe_forward_token_loop(x, wg, b, w1, w3, w2)
    ref, ok = _pair_bruteforce_torch(x, wg, b, w1, w3, w2)
    assert ok.sum() >= len(ok) // 2
    err = np.max(np.abs(y[ok] - ref[ok]))
    assert err <= 1e-5 * np.max(np.abs(ref[ok]))


def test_token_loop_equals_expert_loop_tiny_config():
    cfg = CONFIGS["tiny_fp32"]
    inp = generate(cfg)
    args = (inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    y1, (g1, i1, w1) = oracle.moe_forward_token_loop(*args)
    y2, (g2, i2, w2) = oracle.moe_forward_expert_loop(*args)
    assert np.array_equal(i1, i2) and np.array_equal(w1, w2)
    assert np.max(np.abs(y1 - y2)) <= 1e-6 * np.max(np.abs(y2))


def test_fp32_oracle_within_fp64_shadow():
    cfg = CONFIGS["tiny_fp32"]
    inp = generate(cfg)
    args = (inp["x"], inp["w_gate"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
    y32, (g32, i32, _) = oracle.moe_forward_token_loop(*args)
    y64, (g64, i64, _) = oracle.moe_forward_token_loop(*args, dtype=np.float64)
    srt = np.sort(g64, axis=1)[:, ::-1]
    clear = (srt[:, 1] - srt[:, 2]) > 1e-4
    assert clear.mean() > 0.9
    for t in np.nonzero(clear)[0]:
        assert set(i32[t]) == set(i64[t])
    assert np.max(np.abs(y32[clear] - y64[clear])) <= 1e-5 * np.max(np.abs(y64))


def test_k_equals_E_is_full_softmax_mixture():
    # With E = k = 2 the layer is the softmax-weighted sum of both experts.
    x, wg, w1, w3, w2 = _tiny(9, E=2)
    y, _ = oracle.moe_forward_expert_loop(x, wg, None, w1, w3, w2, k=2)
    g = x.astype(np.float64) @ wg.T.astype(np.float64)
    p = scipy.special.softmax(g, axis=1)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    ref = sum(p[:, e:e + 1] * _torch_swiglu(t(x), t(w1[e]), t(w3[e]), t(w2[e])).numpy() for e in range(2))
    assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_silu_matches_torch():
    z = np.linspace(-30, 30, 2001)
    np.testing.assert_allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------------------
# RMSNorm and the residual sublayer
# ---------------------------------------------------------------------------
def test_rmsnorm_matches_torch_and_closed_form():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((9, 64)) * 3
    gamma = rng.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(z), (64,), torch.from_numpy(gamma), eps=1e-5)
    np.testing.assert_allclose(oracle.rmsnorm_ref(z, gamma, 1e-5, np.float64), ref.numpy(), rtol=1e-12)
    c = 0.01
    row = np.full((1, 32), c)
    out = oracle.rmsnorm_ref(row, None, 1e-5, np.float64)
    np.testing.assert_allclose(out, c / math.sqrt(c * c + 1e-5), rtol=1e-14)


def test_block_is_residual_plus_moe():
    x, wg, w1, w3, w2 = _tiny(4)
    gamma = np.ones(x.shape[1], np.float32)
    out, u, _ = oracle.block_forward_ref(x, gamma, 1e-5, wg, None, w1, w3, np.zeros_like(w2))
    assert np.array_equal(out, x)  # zero down-projection: the sublayer adds exactly 0
    w1e = np.broadcast_to(w1[0], w1.shape).copy()
    w3e = np.broadcast_to(w3[0], w3.shape).copy()
    w2e = np.broadcast_to(w2[0], w2.shape).copy()
    out, _, _ = oracle.block_forward_ref(x, gamma, 1e-5, wg, None, w1e, w3e, w2e)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    un = torch.nn.functional.rms_norm(t(x), (x.shape[1],), eps=1e-5)
    ref = t(x) + _torch_swiglu(un, t(w1[0]), t(w3[0]), t(w2[0]))
    assert np.max(np.abs(out - ref.numpy())) <= 1e-5 * np.max(np.abs(ref.numpy()))


# ---------------------------------------------------------------------------
# load-balancing loss closed forms
# ---------------------------------------------------------------------------
def test_aux_loss_uniform_load_equals_alpha_k():
    E, k, alpha = 8, 2, 0.01
    v = np.array([3.0, 2.0, 0.5, 0.1, -0.2, -1.0, -1.5, -2.0])
    g = np.stack([np.roll(v, s) for s in range(E)])  # each expert at each rank once
    assert abs(oracle.aux_loss_ref([g, g[::-1]], E, k, alpha) - alpha * k) < 1e-12


def test_aux_loss_collapsed_router_equals_alpha_E():
    E, k, alpha = 8, 2, 0.5
    g = np.full((10, E), -1e9)
    g[:, 0] = 4.0
    g[:, 1] = 4.0
    # f_{1,0} = f_{2,1} = 1 and P_0 = P_1 = 1/2  ->  alpha * E * (1/2 + 1/2)
    assert abs(oracle.aux_loss_ref([g], E, k, alpha) - alpha * E) < 1e-12


# ---------------------------------------------------------------------------
# expert Linear biases ("Конфигурация", `bias` key; "Подсчёт параметров")
# ---------------------------------------------------------------------------
def _torch_swiglu_linear(u, w1, w3, w2, b1, b3, b2):
    """The biased expert through torch's own Linear (F.linear adds the bias)."""
    F = torch.nn.functional
    return F.linear(F.silu(F.linear(u, w1, b1)) * F.linear(u, w3, b3), w2, b2)


def _tiny_bias(seed, E=8, d=16, d_ff=24):
    rng = np.random.default_rng(100 + seed)
    return (rng.standard_normal((E, d_ff)).astype(np.float32) * 0.5,
            rng.standard_normal((E, d_ff)).astype(np.float32) * 0.5,
            rng.standard_normal((E, d)).astype(np.float32) * 0.5)


def _pair_bruteforce_torch_bias(x, wg, b, w1, w3, w2, eb):
    """As _pair_bruteforce_torch, each expert evaluated by torch's biased Linear."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    X, WG = t(x), t(wg)
    G = X @ WG.T + (t(b) if b is not None else 0)
    T = G.shape[0]
    y = torch.zeros_like(X)
    ok = np.ones(T, bool)
    for tt in range(T):
        gt = G[tt]
        srt = torch.sort(gt, descending=True).values
        ok[tt] = bool(srt[1] - srt[2] > 1e-3)
        i, j = _pair_argmax(gt.tolist())
        wts = torch.softmax(torch.stack([gt[i], gt[j]]), dim=0)
        for wgt, e in zip(wts, (i, j)):
            y[tt] += wgt * _torch_swiglu_linear(X[tt:tt + 1], t(w1[e]), t(w3[e]), t(w2[e]),
                                                t(eb[0][e]), t(eb[1][e]), t(eb[2][e]))[0]
    return y.numpy(), ok


@pytest.mark.parametrize("seed", [0, 1])
def test_biased_experts_equal_28_pair_bruteforce(seed):
    x, wg, w1, w3, w2 = _tiny(seed)
    eb = _tiny_bias(seed)
    y1, _ = oracle.moe_forward_token_loop(x, wg, None, w1, w3, w2, eb=eb)
    y2, _ = oracle.moe_forward_expert_loop(x, wg, None, w1, w3, w2, eb=eb)
    ref, ok = _pair_bruteforce_torch_bias(x, wg, None, w1, w3, w2, eb)
    assert ok.sum() >= len(ok) // 2
    for y in (y1, y2):
        assert np.max(np.abs(y[ok] - ref[ok])) <= 1e-5 * np.max(np.abs(ref[ok]))


def test_biased_identity_when_all_experts_equal():
    x, wg, w1, w3, w2 = _tiny(2)
    b1, b3, b2 = _tiny_bias(2)
    rep = lambda a: np.broadcast_to(a[5], a.shape).copy()
    W1, W3, W2, B1, B3, B2 = map(rep, (w1, w3, w2, b1, b3, b2))
    y, _ = oracle.moe_forward_expert_loop(x, wg, None, W1, W3, W2, eb=(B1, B3, B2))
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    dense = _torch_swiglu_linear(t(x), t(W1[0]), t(W3[0]), t(W2[0]), t(B1[0]), t(B3[0]), t(B2[0])).numpy()
    assert np.max(np.abs(y - dense)) <= 1e-5 * np.max(np.abs(dense))


def test_biases_closed_forms():
    """Zero weights leave only the biases: with W2 = 0 the layer is sum_s w_s b2[e_s];
    with W1 = W3 = 0 every row of expert e is SiLU(b1[e]) * b3[e] through W2, plus b2[e]."""
    x, wg, w1, w3, w2 = _tiny(3)
    b1, b3, b2 = _tiny_bias(3)
    _, idx, w = oracle.route_ref(x, wg, None)
    y, _ = oracle.moe_forward_expert_loop(x, wg, None, w1, w3, np.zeros_like(w2), eb=(b1, b3, b2))
    ref = sum(w[:, s:s + 1].astype(np.float64) * b2[idx[:, s]] for s in range(2))
    assert np.max(np.abs(y - ref)) <= 1e-6
    y, _ = oracle.moe_forward_expert_loop(x, wg, None, np.zeros_like(w1), np.zeros_like(w3), w2, eb=(b1, b3, b2))
    h = scipy.special.expit(b1.astype(np.float64)) * b1 * b3  # [E, d_ff]
    per_e = np.einsum("ef,edf->ed", h, w2.astype(np.float64)) + b2
    ref = sum(w[:, s:s + 1].astype(np.float64) * per_e[idx[:, s]] for s in range(2))
    assert np.max(np.abs(y - ref)) <= 1e-5 * np.max(np.abs(ref))


def test_zero_biases_equal_no_biases():
    x, wg, w1, w3, w2 = _tiny(4)
    z = (np.zeros((8, 24), np.float32), np.zeros((8, 24), np.float32), np.zeros((8, 16), np.float32))
    y0, _ = oracle.moe_forward_expert_loop(x, wg, None, w1, w3, w2)
    y1, _ = oracle.moe_forward_expert_loop(x, wg, None, w1, w3, w2, eb=z)
    assert np.array_equal(y0, y1)
    # each bias may be absent on its own
    y2, _ = oracle.moe_forward_expert_loop(x, wg, None, w1, w3, w2, eb=(None, z[1], None))
    assert np.array_equal(y0, y2)


def _mut_bias_after_silu(u, w1_e, w3_e, w2_e, dtype=np.float32, b1_e=None, b3_e=None, b2_e=None):
    u = moe_ref.widen(u, dtype)
    a = moe_ref.silu(u @ moe_ref.widen(w1_e, dtype).T) + b1_e
    h = a * (u @ moe_ref.widen(w3_e, dtype).T + b3_e)
    return (h @ moe_ref.widen(w2_e, dtype).T + b2_e).astype(dtype)


def _mut_down_bias_dropped(u, w1_e, w3_e, w2_e, dtype=np.float32, b1_e=None, b3_e=None, b2_e=None):
    return _orig_expert(u, w1_e, w3_e, w2_e, dtype, b1_e, b3_e, None)


@pytest.mark.parametrize("name,mutant", [
    ("gate bias after SiLU", _mut_bias_after_silu),
    ("down bias dropped", _mut_down_bias_dropped),
])
def test_planted_bias_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(moe_ref, "expert_swiglu", mutant)
    x, wg, w1, w3, w2 = _tiny(0)
    eb = _tiny_bias(0)
    y, _ = moe_ref.moe_forward_token_loop(x, wg, None, w1, w3, w2, eb=eb)
    monkeypatch.undo()
    ref, ok = _pair_bruteforce_torch_bias(x, wg, None, w1, w3, w2, eb)
    assert np.max(np.abs(y[ok] - ref[ok])) > 1e-3 * np.max(np.abs(ref[ok])), name


# ---------------------------------------------------------------------------
# planted mistakes: a mutated copy of the oracle must fail a pin
# ---------------------------------------------------------------------------
def _mut_silu_sign(z):
    return z / (1 + np.exp(z))


def _mut_swap_gate_up(u, w1_e, w3_e, w2_e, dtype=np.float32, *biases):
    return _orig_expert(u, w3_e, w1_e, w2_e, dtype)


def _mut_transpose_down(u, w1_e, w3_e, w2_e, dtype=np.float32, *biases):
    u = moe_ref.widen(u, dtype)
    h = moe_ref.silu(u @ moe_ref.widen(w1_e, dtype).T) * (u @ moe_ref.widen(w3_e, dtype).T)
    w2 = moe_ref.widen(w2_e, dtype)
    return (h @ w2.reshape(w2.shape[1], w2.shape[0])).astype(dtype)


def _mut_smallest(g, k=2):
    return np.argsort(g, axis=1, kind="stable")[:, :k].astype(np.int32)


def _mut_swap_slots(g, idx, dtype=np.float32):
    return _orig_softmax(g, idx, dtype)[:, ::-1].copy()


def _mut_no_renorm(g, idx, dtype=np.float32):
    sel = np.take_along_axis(g.astype(dtype), idx.astype(np.int64), axis=1)
    return np.exp(sel).astype(dtype)


_orig_expert = moe_ref.expert_swiglu
_orig_softmax = moe_ref.topk_softmax


@pytest.mark.parametrize("name,target,mutant", [
    ("silu sign", "silu", _mut_silu_sign),
    ("gate/up swapped", "expert_swiglu", _mut_swap_gate_up),
    ("down projection mis-laid", "expert_swiglu", _mut_transpose_down),
    ("bottom-2 instead of top-2", "top2", _mut_smallest),
    ("weights on the wrong slots", "topk_softmax", _mut_swap_slots),
    ("softmax not normalised", "topk_softmax", _mut_no_renorm),
])
def test_planted_mistake_is_caught(monkeypatch, name, target, mutant):
    monkeypatch.setattr(moe_ref, target, mutant)
    x, wg, w1, w3, w2 = _tiny(0, d=16, d_ff=16)
    y, _ = moe_ref.moe_forward_token_loop(x, wg, None, w1, w3, w2)
    monkeypatch.undo()
    ref, ok = _pair_bruteforce_torch(x, wg, None, w1, w3, w2)
    err = np.max(np.abs(y[ok] - ref[ok]))
    assert err > 1e-3 * np.max(np.abs(ref[ok])), name


# ---------------------------------------------------------------------------
# gather form of the combine == the pages' index-add form
# ---------------------------------------------------------------------------
def test_gather_combine_equals_index_add():
    cfg = CONFIGS["tiny_fp32"]
    inp = generate(cfg)
    y_ref, (g, idx, w) = oracle.moe_forward_expert_loop(inp["x"], inp["w_gate"], None, inp["w1"], inp["w3"],
                                                        inp["w2"])
    off, st, inv = oracle.dispatch_ref(idx, cfg.E)
    rows = oracle.expert_rows_ref(inp["x"], st, off, inp["w1"], inp["w3"], inp["w2"])
    y = oracle.combine_ref(rows, inv, w)
    assert np.max(np.abs(y - y_ref)) <= 1e-6 * np.max(np.abs(y_ref))
    res = np.ones_like(y)
    np.testing.assert_allclose(oracle.combine_ref(rows, inv, w, res) - y, 1.0, atol=1e-5)


def test_router_stats_are_distributions():
    rng = np.random.default_rng(11)
    g = [rng.standard_normal((50, 8)) for _ in range(3)]
    mask = rng.uniform(size=50) > 0.3
    f, P = oracle.router_stats_ref(g, 8, 2, mask)
    np.testing.assert_allclose(f.sum(axis=1), 1.0, rtol=1e-12)   # each slot picks one expert per token
    np.testing.assert_allclose(P.sum(), 1.0, rtol=1e-12)          # mean of distributions
    assert np.all(f[0] + f[1] <= 1.0 + 1e-12)                     # an expert fills at most one slot per token
    f0, P0 = oracle.router_stats_ref(g, 8, 2, np.zeros(50, bool))
    assert not f0.any() and not P0.any()


# ---------------------------------------------------------------------------
# load-balancing loss against HuggingFace's Mixtral ("Load-balancing loss": the
# page's loss agrees with HF's load_balancing_loss_func up to float; P_i is
# the mean of the router's softmax over all E experts)
# ---------------------------------------------------------------------------
def _hf_lb_loss(logits_per_layer, E, k, mask=None):
    from transformers.models.mixtral.modeling_mixtral import load_balancing_loss_func

    g = tuple(torch.from_numpy(np.asarray(a, np.float64)) for a in logits_per_layer)
    m = None if mask is None else torch.from_numpy(np.asarray(mask, np.int64))[None, :]
    return float(load_balancing_loss_func(g, E, k, m))


@pytest.mark.parametrize("E,k,layers,masked", [(8, 2, 1, False), (8, 2, 3, True), (16, 4, 2, False),
                                                (4, 1, 2, True), (64, 6, 1, True)])
def test_aux_loss_matches_hf_load_balancing_loss(E, k, layers, masked):
    rng = np.random.default_rng(E * 10 + k)
    T = 97
    # non-uniform logits: a per-expert offset makes P_i differ from the top-k shares
    g = [rng.standard_normal((T, E)) * 1.5 + np.linspace(-1, 2, E)[None, :] for _ in range(layers)]
    mask = (rng.uniform(size=T) > 0.25) if masked else None
    want = _hf_lb_loss(g, E, k, mask)
    got = oracle.aux_loss_ref(g, E, k, alpha=1.0, token_mask=mask)
    # HF averages the one-hot top-k mask in float32 (f_{s,i} rounded to fp32)
    assert abs(got - want) <= 1e-6 * abs(want)


def test_router_stats_P_is_mean_full_softmax():
    rng = np.random.default_rng(3)
    g = [rng.standard_normal((40, 8)) * 2 for _ in range(2)]
    mask = rng.uniform(size=40) > 0.3
    _, P = oracle.router_stats_ref(g, 8, 2, mask)
    rows = np.concatenate([a[mask] for a in g])
    np.testing.assert_allclose(P, scipy.special.softmax(rows, axis=1).mean(axis=0), rtol=1e-13)


def _mut_stats_topk_P(logits_per_layer, E, k, token_mask=None, dtype=np.float64):
    """Planted mistake: P_i from the renormalised top-k weights instead of the full softmax."""
    f, _ = _orig_stats(logits_per_layer, E, k, token_mask, dtype)
    G = np.concatenate([np.asarray(a, dtype)[np.asarray(token_mask, bool)] if token_mask is not None
                        else np.asarray(a, dtype) for a in logits_per_layer])
    idx = moe_ref.top2(G, k)
    w = moe_ref.topk_softmax(G, idx, dtype)
    P = np.zeros((G.shape[0], E), dtype)
    np.put_along_axis(P, idx.astype(np.int64), w, axis=1)
    return f, P.mean(axis=0)


_orig_stats = moe_ref.router_stats_ref


def test_planted_topk_P_fails_hf_pin(monkeypatch):
    monkeypatch.setattr(moe_ref, "router_stats_ref", _mut_stats_topk_P)
    rng = np.random.default_rng(80)
    g = [rng.standard_normal((97, 8)) * 1.5 + np.linspace(-1, 2, 8)[None, :]]
    got = moe_ref.aux_loss_ref(g, 8, 2, alpha=1.0)
    monkeypatch.undo()
    want = _hf_lb_loss(g, 8, 2)
    assert abs(got - want) > 1e-2 * abs(want)
    # the two closed-form pins cannot tell this mutant apart (both hold for it too)
    v = np.array([3.0, 2.0, 0.5, 0.1, -0.2, -1.0, -1.5, -2.0])
    u = np.stack([np.roll(v, s) for s in range(8)])
    assert abs(_mut_stats_topk_P([u], 8, 2)[1].sum() - 1.0) < 1e-12


# ---------------------------------------------------------------------------
# the whole layer against HuggingFace's MixtralSparseMoeBlock ("Mixtral" page,
# "Загрузка весов HuggingFace": w1 / w3 / w2 map to gate / up / down, and the
# page's library reproduces HF's logits).  HF computes the softmax over all E
# logits, keeps the top k and renormalises them: the same weights as a
# softmax over the kept logits.
# ---------------------------------------------------------------------------
def _hf_moe_block(x, wg, w1, w3, w2, k):
    from transformers import MixtralConfig
    from transformers.models.mixtral import modeling_mixtral as mm

    E, d_ff, d = w1.shape
    cfg = MixtralConfig(hidden_size=d, intermediate_size=d_ff, num_local_experts=E, num_experts_per_tok=k)
    blk = mm.MixtralSparseMoeBlock(cfg).double().eval()
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    with torch.no_grad():
        blk.gate.weight.copy_(t(wg))
        blk.experts.gate_up_proj.copy_(torch.cat([t(w1), t(w3)], dim=1))
        blk.experts.down_proj.copy_(t(w2))
        return blk(t(x)[None])[0].numpy()


@pytest.mark.parametrize("E,k,T,d,d_ff", [(8, 2, 40, 16, 24), (16, 2, 33, 32, 16), (8, 4, 20, 16, 32),
                                           (4, 1, 25, 8, 16)])
def test_layer_matches_hf_mixtral_sparse_moe_block(E, k, T, d, d_ff):
    rng = np.random.default_rng(E * 100 + k)
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, d)) * 0.5
    w1 = rng.standard_normal((E, d_ff, d)) / np.sqrt(d)
    w3 = rng.standard_normal((E, d_ff, d)) / np.sqrt(d)
    w2 = rng.standard_normal((E, d, d_ff)) / np.sqrt(d_ff)
    want = _hf_moe_block(x, wg, w1, w3, w2, k)
    g = x @ wg.T
    s = np.sort(g, axis=1)[:, ::-1]
    clear = (s[:, k - 1] - s[:, k]) > 1e-6 if k < E else np.ones(T, bool)
    assert clear.mean() > 0.9
    # HF takes the router softmax in float32 even in a float64 module: weights
    # carry about 2^-24 of relative error, the rest is float64.
    for fn in (oracle.moe_forward_expert_loop, oracle.moe_forward_token_loop):
        got, _ = fn(x, wg, None, w1, w3, w2, k=k, dtype=np.float64)
        assert np.max(np.abs(got[clear] - want[clear])) <= 1e-6 * np.max(np.abs(want))


def test_planted_gate_up_swap_fails_hf_pin(monkeypatch):
    monkeypatch.setattr(moe_ref, "expert_swiglu", _mut_swap_gate_up)
    rng = np.random.default_rng(5)
    T, d, d_ff, E = 30, 16, 24, 8
    x, wg = rng.standard_normal((T, d)), rng.standard_normal((E, d)) * 0.5
    w1, w3 = rng.standard_normal((E, d_ff, d)) / 4, rng.standard_normal((E, d_ff, d)) / 4
    w2 = rng.standard_normal((E, d, d_ff)) / 5
    got, _ = moe_ref.moe_forward_expert_loop(x, wg, None, w1, w3, w2, dtype=np.float64)
    monkeypatch.undo()
    want = _hf_moe_block(x, wg, w1, w3, w2, 2)
    assert np.max(np.abs(got - want)) > 1e-2 * np.max(np.abs(want))
