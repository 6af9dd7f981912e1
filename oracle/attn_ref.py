"""Plain CPU reference of the attention sublayer around the MoE: GQA with RoPE.

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the benchmark's
CPU-baseline leg; never by the product path.

Source: "Mixtral" textbook page, section "Прямой проход в формулах" (forward
pass in formulas), the block equation U = H + GQA(RMSNorm_1(H)) and the GQA
equations: for the normalised input X, query head h and its K/V group
kappa(h) = floor(h / r), r = H / G,
    Q_h = RoPE(X W_Q^h),  K_c = RoPE(X W_K^c),  V_c = X W_V^c,
    O_h = softmax(Q_h K_kappa(h)^T / sqrt(d_h) + M) V_kappa(h),
    GQA(X) = [O_0; ...; O_{H-1}] W_O,
with M the causal mask (0 on and below the diagonal, -inf above).  The same
page lists the base of the rotation frequencies (rope_theta: 1e6 in Mixtral
8x7B, 1e4 by default in the library).

Readings where the pages are silent (each listed in the design notes):
  * RoPE itself is defined in another chapter.  The page's HuggingFace loader
    permutes the rows of q_proj / k_proj per head, which converts HF's
    half-split rotation into the interleaved one, so the library rotates
    adjacent pairs: for head dimension pair (2i, 2i+1) at position p, with
    theta_i = rope_theta ** (-2i / d_h), the pair is multiplied, as the
    complex number x_{2i} + j x_{2i+1}, by e^{j p theta_i}.
  * Positions of a sequence of T new tokens are pos0 .. pos0 + T - 1.
  * Weights are nn.Linear layout: W_Q [H*d_h, d], W_K, W_V [G*d_h, d],
    W_O [d, H*d_h]; head h of Q is columns h*d_h .. h*d_h + d_h - 1 of X W_Q^T.
  * No Linear biases (Mixtral 8x7B has none), no dropout, no sliding window
    (Mixtral attends densely).

Precision: fp32 by default, fp64 with dtype=np.float64 for the error-bound pins.
"""
from __future__ import annotations

import numpy as np

from .moe_ref import rmsnorm_ref, widen


def rope_ref(x, positions, theta: float, dtype=np.float32) -> np.ndarray:
    """Rotate every head vector of x [T, n_heads, d_h] by its token's position.

    Pair (2i, 2i+1) turns by the angle p * theta**(-2i/d_h)."""
    x = widen(x, dtype)
    T, nh, dh = x.shape
    i = np.arange(dh // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / dh)                                   # [d_h/2]
    ang = np.asarray(positions, np.float64)[:, None] * inv_freq[None, :]  # [T, d_h/2]
    c = np.cos(ang).astype(dtype)[:, None, :]
    s = np.sin(ang).astype(dtype)[:, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def gqa_attention_ref(q, k, v, causal: bool = True, dtype=np.float32) -> np.ndarray:
    """O_h = softmax(Q_h K_kappa(h)^T / sqrt(d_h) + M) V_kappa(h) for every query head.

    q [T, H, d_h], k and v [T_k, G, d_h] (already rotated); returns [T, H, d_h].
    With causal, query t (the last T of the T_k positions) sees keys up to
    its own position."""
    q, k, v = widen(q, dtype), widen(k, dtype), widen(v, dtype)
    T, H, dh = q.shape
    Tk, G, _ = k.shape
    r = H // G
    out = np.empty((T, H, dh), dtype=dtype)
    mask = np.zeros((T, Tk), dtype=dtype)
    if causal:
        qpos = np.arange(Tk - T, Tk)[:, None]
        mask = np.where(np.arange(Tk)[None, :] > qpos, -np.inf, 0.0).astype(dtype)
    scale = np.asarray(1.0 / np.sqrt(dh), dtype)
    for h in range(H):
        c = h // r
        s = (q[:, h, :] @ k[:, c, :].T) * scale + mask
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, c, :]
    return out


def attention_sublayer_ref(h, gamma, eps, wq, wk, wv, wo, H: int, G: int, rope_theta: float,
                           pos0: int = 0, dtype=np.float32):
    """U = H + GQA(RMSNorm_1(H)) for one sequence of T tokens (causal, positions pos0 ..).

    Returns (u_out [T, d], x [T, d] normalised input, (q, k, v) rotated heads,
    o [T, H, d_h] attention output before W_O)."""
    Hs = widen(h, dtype)
    T, d = Hs.shape
    x = rmsnorm_ref(Hs, gamma, eps, dtype)
    WQ, WK, WV, WO = (widen(w, dtype) for w in (wq, wk, wv, wo))
    dh = WQ.shape[0] // H
    pos = np.arange(pos0, pos0 + T)
    q = rope_ref((x @ WQ.T).reshape(T, H, dh), pos, rope_theta, dtype)
    k = rope_ref((x @ WK.T).reshape(T, G, dh), pos, rope_theta, dtype)
    v = (x @ WV.T).reshape(T, G, dh)
    o = gqa_attention_ref(q, k, v, True, dtype)
    u = Hs + o.reshape(T, H * dh) @ WO.T
    return u.astype(dtype, copy=False), x, (q, k, v), o
