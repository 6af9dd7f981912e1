"""Pins of the attention oracle (GQA with RoPE, "Mixtral" page, "Прямой проход в
формулах") to facts fixed by mathematics and by independent library routines:
the complex-number form of the rotation, its relative-position property,
torch's scaled_dot_product_attention with K/V heads repeated per group,
causality, and planted mistakes that must fail those pins."""
import numpy as np
import pytest
import torch

import oracle
from oracle import attn_ref


def _rng(seed):
    return np.random.default_rng(1000 + seed)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def _rope_complex(x, pos, theta):
    """Pair (2i, 2i+1) as the complex number x_2i + j x_2i+1, times e^{j p theta^(-2i/d_h)}."""
    x = np.asarray(x, np.float64)
    dh = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    ang = np.asarray(pos, np.float64)[:, None, None] * theta ** (-2.0 * np.arange(dh // 2) / dh)
    w = z * np.exp(1j * ang)
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = w.real, w.imag
    return out


@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_rope_equals_complex_rotation(theta):
    x = _rng(0).standard_normal((9, 3, 16))
    pos = np.arange(100, 109)
    got = attn_ref.rope_ref(x, pos, theta, np.float64)
    assert np.max(np.abs(got - _rope_complex(x, pos, theta))) < 1e-12


def test_rope_position_zero_is_identity_and_norm_is_kept():
    x = _rng(1).standard_normal((4, 2, 32))
    assert np.array_equal(attn_ref.rope_ref(x, np.zeros(4), 1e6, np.float64), x)
    y = attn_ref.rope_ref(x, np.arange(4) * 777, 1e6, np.float64)
    n = lambda a: np.hypot(a[..., 0::2], a[..., 1::2])
    assert np.max(np.abs(n(y) - n(x))) < 1e-12


def test_rope_scores_depend_on_relative_position_only():
    q = _rng(2).standard_normal((1, 1, 64))
    k = _rng(3).standard_normal((1, 1, 64))
    dot = lambda m, n: float(np.sum(attn_ref.rope_ref(q, [m], 1e6, np.float64) *
                                    attn_ref.rope_ref(k, [n], 1e6, np.float64)))
    for shift in (1, 37, 4000):
        assert abs(dot(10, 3) - dot(10 + shift, 3 + shift)) < 1e-9


# ---------------------------------------------------------------------------
# GQA attention against torch's scaled_dot_product_attention
# ---------------------------------------------------------------------------
def _sdpa(q, k, v, causal=True):
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    Q, K, V = t(q).transpose(0, 1), t(k).transpose(0, 1), t(v).transpose(0, 1)  # [heads, T, d_h]
    r = Q.shape[0] // K.shape[0]
    K, V = K.repeat_interleave(r, dim=0), V.repeat_interleave(r, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal)
    return o.transpose(0, 1).numpy()


@pytest.mark.parametrize("T,H,G,dh", [(17, 8, 2, 16), (33, 4, 4, 8), (20, 6, 1, 32), (1, 4, 2, 16)])
def test_gqa_matches_torch_sdpa(T, H, G, dh):
    rng = _rng(T + H)
    q, k, v = rng.standard_normal((T, H, dh)), rng.standard_normal((T, G, dh)), rng.standard_normal((T, G, dh))
    got = attn_ref.gqa_attention_ref(q, k, v, True, np.float64)
    assert np.max(np.abs(got - _sdpa(q, k, v))) < 1e-12
    got32 = attn_ref.gqa_attention_ref(q, k, v, True)
    assert np.max(np.abs(got32 - got)) < 1e-5


def test_gqa_is_causal():
    rng = _rng(5)
    q, k, v = rng.standard_normal((12, 4, 8)), rng.standard_normal((12, 2, 8)), rng.standard_normal((12, 2, 8))
    a = attn_ref.gqa_attention_ref(q, k, v, True, np.float64)
    k2, v2 = k.copy(), v.copy()
    k2[7:] += 3.0
    v2[7:] -= 5.0
    b = attn_ref.gqa_attention_ref(q, k2, v2, True, np.float64)
    assert np.array_equal(a[:7], b[:7]) and not np.allclose(a[7:], b[7:])
    assert np.allclose(a[0], np.repeat(v[0], 2, axis=0))  # the first query sees only key 0


# ---------------------------------------------------------------------------
# the whole sublayer against a torch composition
# ---------------------------------------------------------------------------
def _sublayer_torch(h, gamma, eps, wq, wk, wv, wo, H, G, theta, pos0):
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    F = torch.nn.functional
    X = F.rms_norm(t(h), (h.shape[1],), t(gamma), eps)
    T = h.shape[0]
    dh = wq.shape[0] // H
    pos = np.arange(pos0, pos0 + T)
    q = _rope_complex(F.linear(X, t(wq)).reshape(T, H, dh).numpy(), pos, theta)
    k = _rope_complex(F.linear(X, t(wk)).reshape(T, G, dh).numpy(), pos, theta)
    v = F.linear(X, t(wv)).reshape(T, G, dh).numpy()
    o = _sdpa(q, k, v)
    return (t(h) + F.linear(t(o.reshape(T, H * dh)), t(wo))).numpy()


def test_attention_sublayer_matches_torch_composition():
    rng = _rng(7)
    T, d, H, G, dh = 21, 64, 8, 2, 16
    h = rng.standard_normal((T, d)).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, d).astype(np.float32)
    wq = (rng.standard_normal((H * dh, d)) / 8).astype(np.float32)
    wk = (rng.standard_normal((G * dh, d)) / 8).astype(np.float32)
    wv = (rng.standard_normal((G * dh, d)) / 8).astype(np.float32)
    wo = (rng.standard_normal((d, H * dh)) / 12).astype(np.float32)
    ref = _sublayer_torch(h, gamma, 1e-5, wq, wk, wv, wo, H, G, 1e6, 5)
    got, *_ = attn_ref.attention_sublayer_ref(h, gamma, 1e-5, wq, wk, wv, wo, H, G, 1e6, pos0=5)
    assert np.max(np.abs(got - ref)) < 1e-4 * np.max(np.abs(ref))
    got64, *_ = attn_ref.attention_sublayer_ref(h, gamma, 1e-5, wq, wk, wv, wo, H, G, 1e6, pos0=5, dtype=np.float64)
    assert np.max(np.abs(got64 - ref)) < 1e-12 * np.max(np.abs(ref))


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
def _rope_half_split(x, positions, theta, dtype=np.float32):
    x = np.asarray(x, dtype)
    dh = x.shape[-1]
    ang = np.asarray(positions, np.float64)[:, None] * theta ** (-2.0 * np.arange(dh // 2) / dh)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :dh // 2], x[..., dh // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1).astype(dtype)


def _attn_sees_next(q, k, v, causal=True, dtype=np.float32):
    q, k, v = (np.asarray(a, dtype) for a in (q, k, v))
    T, H, dh = q.shape
    r = H // k.shape[1]
    out = np.empty_like(q)
    mask = np.where(np.arange(T)[None, :] > np.arange(T)[:, None] + 1, -np.inf, 0.0)
    for h in range(H):
        s = q[:, h] @ k[:, h // r].T / np.sqrt(dh) + mask
        p = np.exp(s - s.max(1, keepdims=True))
        out[:, h] = (p / p.sum(1, keepdims=True)) @ v[:, h // r]
    return out


def test_planted_rope_pairing_is_caught():
    x = _rng(8).standard_normal((5, 2, 16))
    pos = np.arange(3, 8)
    assert np.max(np.abs(_rope_half_split(x, pos, 1e4, np.float64) - _rope_complex(x, pos, 1e4))) > 1e-2


@pytest.mark.parametrize("mutant", ["sees_next", "wrong_group"])
def test_planted_attention_mistake_is_caught(mutant):
    rng = _rng(9)
    q, k, v = rng.standard_normal((10, 8, 8)), rng.standard_normal((10, 2, 8)), rng.standard_normal((10, 2, 8))
    if mutant == "sees_next":
        got = _attn_sees_next(q, k, v, True, np.float64)
    else:
        G, H = 2, 8
        kk = np.stack([k[:, h % G] for h in range(H)], axis=1)
        vv = np.stack([v[:, h % G] for h in range(H)], axis=1)
        got = attn_ref.gqa_attention_ref(q, kk, vv, True, np.float64)
    assert np.max(np.abs(got - _sdpa(q, k, v))) > 1e-2


# ---------------------------------------------------------------------------
# RoPE frequency schedule and pairing against HuggingFace's Mixtral.  The
# "Mixtral" page ("Загрузка весов HuggingFace") loads HF checkpoints by
# reordering the rows of q_proj (per query head) and k_proj (per K/V head);
# with that reordering the library's rotation must reproduce HF's.  HF's
# rotary module and attention run here offline on a random tiny config.
# ---------------------------------------------------------------------------
def _hf_rows_to_interleaved(w, n_heads, dh):
    """Per head, HF's rotation partners (j, j + dh/2) become rows (2j, 2j + 1)."""
    w = np.asarray(w)
    out = np.empty_like(w)
    for h in range(n_heads):
        blk = w[h * dh:(h + 1) * dh]
        dst = out[h * dh:(h + 1) * dh]
        dst[0::2] = blk[:dh // 2]
        dst[1::2] = blk[dh // 2:]
    return out


def _hf_mixtral(H, G, dh, d, theta):
    from transformers import MixtralConfig
    from transformers.models.mixtral import modeling_mixtral as mm

    cfg = MixtralConfig(hidden_size=d, num_attention_heads=H, num_key_value_heads=G, head_dim=dh, rope_theta=theta,
                        intermediate_size=32, num_local_experts=4)
    cfg._attn_implementation = "sdpa"
    return cfg, mm


def _rope_by_hf(x, pos, theta):
    """x [T, n, dh] rotated by HF's MixtralRotaryEmbedding + apply_rotary_pos_emb (half-split pairs)."""
    T, n, dh = x.shape
    cfg, mm = _hf_mixtral(n, n, dh, n * dh, theta)
    rot = mm.MixtralRotaryEmbedding(cfg)
    X = torch.from_numpy(np.asarray(x, np.float64)).transpose(0, 1)[None]  # [1, n, T, dh]
    cos, sin = rot(X, torch.as_tensor(np.asarray(pos))[None])
    out, _ = mm.apply_rotary_pos_emb(X, X, cos, sin)
    return out[0].transpose(0, 1).numpy()


def _interleave_cols(y):
    """Columns of a half-split head vector in the interleaved order (j -> 2j, j + dh/2 -> 2j + 1)."""
    dh = y.shape[-1]
    out = np.empty_like(y)
    out[..., 0::2], out[..., 1::2] = y[..., :dh // 2], y[..., dh // 2:]
    return out


@pytest.mark.parametrize("theta,dh", [(1e4, 16), (1e6, 32), (1e6, 128)])
def test_rope_matches_hf_mixtral_after_row_permutation(theta, dh):
    """rope_ref of the permuted projection == HF's rotation of the HF projection,
    column j of HF's head landing on 2j and column j + dh/2 on 2j + 1.  This fixes
    both the pairing and the schedule theta^(-2i/d_h), including i = 0."""
    rng = _rng(20 + dh)
    T, n = 11, 3
    y_hf = rng.standard_normal((T, n, dh))
    pos = np.arange(40, 40 + T)
    want = _interleave_cols(_rope_by_hf(y_hf, pos, theta))
    got = attn_ref.rope_ref(_interleave_cols(y_hf), pos, theta, np.float64)
    # HF forms the angles in float32: about p * 2^-24 rad of error per pair
    assert np.max(np.abs(got - want)) < 1e-4 * np.max(np.abs(want))


def test_attention_matches_hf_mixtral_attention():
    """The oracle's GQA with RoPE and W_O (no norm, no residual) on HF weights whose
    q_proj / k_proj rows are reordered as the page's loader does == HF's
    MixtralAttention (sdpa, causal) on the original weights."""
    rng = _rng(30)
    T, d, H, G, dh, theta, pos0 = 13, 64, 4, 2, 16, 1e6, 7
    cfg, mm = _hf_mixtral(H, G, dh, d, theta)
    att = mm.MixtralAttention(cfg, 0).double()
    wq = rng.standard_normal((H * dh, d)) / 8
    wk = rng.standard_normal((G * dh, d)) / 8
    wv = rng.standard_normal((G * dh, d)) / 8
    wo = rng.standard_normal((d, H * dh)) / 8
    with torch.no_grad():
        for name, w in (("q_proj", wq), ("k_proj", wk), ("v_proj", wv), ("o_proj", wo)):
            getattr(att, name).weight.copy_(torch.from_numpy(w))
        x = torch.from_numpy(rng.standard_normal((1, T, d)))
        cos, sin = mm.MixtralRotaryEmbedding(cfg)(x, torch.arange(pos0, pos0 + T)[None])
        want, _ = att(x, (cos, sin), None)
    want = want[0].numpy()
    X = x[0].numpy()
    wq_l, wk_l = _hf_rows_to_interleaved(wq, H, dh), _hf_rows_to_interleaved(wk, G, dh)
    pos = np.arange(pos0, pos0 + T)
    q = attn_ref.rope_ref((X @ wq_l.T).reshape(T, H, dh), pos, theta, np.float64)
    k = attn_ref.rope_ref((X @ wk_l.T).reshape(T, G, dh), pos, theta, np.float64)
    v = (X @ wv.T).reshape(T, G, dh)
    got = attn_ref.gqa_attention_ref(q, k, v, True, np.float64).reshape(T, H * dh) @ wo.T
    assert np.max(np.abs(got - want)) < 1e-5 * np.max(np.abs(want))


def _rope_wrong_schedule(x, positions, theta, dtype=np.float32):
    """Planted mistake: theta^(-i/d_h) instead of theta^(-2i/d_h)."""
    x = np.asarray(x, dtype)
    dh = x.shape[-1]
    ang = np.asarray(positions, np.float64)[:, None] * theta ** (-1.0 * np.arange(dh // 2) / dh)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


@pytest.mark.parametrize("mutant", [_rope_wrong_schedule, _rope_half_split])
def test_planted_rope_mistake_fails_hf_pin(monkeypatch, mutant):
    monkeypatch.setattr(attn_ref, "rope_ref", mutant)
    rng = _rng(21)
    y_hf = rng.standard_normal((11, 3, 32))
    pos = np.arange(40, 51)
    want = _interleave_cols(_rope_by_hf(y_hf, pos, 1e6))
    got = attn_ref.rope_ref(_interleave_cols(y_hf), pos, 1e6, np.float64)
    assert np.max(np.abs(got - want)) > 1e-2 * np.max(np.abs(want))
