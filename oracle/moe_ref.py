"""Plain CPU reference of the Mixtral sparse MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the benchmark's
CPU-baseline leg; never by the product path.

Sources (all on the pages this project follows):
  [MIX-F]  "Mixtral" textbook page, section "Прямой проход в формулах"
           (forward pass in formulas): the MoE equation g = u W_r,
           S = TopK(g, k), w_i = e^{g_i} / sum_{j in S} e^{g_j},
           MoE(u) = sum_{i in S} w_i (SiLU(u W_gate^i) * u W_up^i) W_down^i;
           the RMSNorm equation and the pre-LN block equation
           H = U + MoE(RMSNorm_2(U)).
  [MIX-C]  same page, section "Научный вклад" (contribution): the layer
           formula y = sum_i Softmax(Top2(x W_g))_i SwiGLU_i(x), Top2 keeps the
           two largest logits and sets the others to -inf.
  [MIX-IN] same page, section "MoE изнутри" (MoE inside): router is a Linear
           layer, top-k then a softmax over the k kept logits in float32, each
           expert sees only its tokens, output is the weighted sum.
  [MIX-A]  same page, section "Алгоритм" (algorithm): an outer loop over
           experts, each expert applied to the tokens that selected it (in
           token order), experts without tokens skipped, the weighted outputs
           accumulated at their tokens; every token gets exactly k terms
           (dropless), and the result is checked against a token-by-token loop.
  [MIX-LB] same page, section "Load-balancing loss".
  [MIX-HF] same page, section "Загрузка весов HuggingFace": router w1/w3/w2
           map to gate/up/down.
  [MIX-B]  same page, section "Конфигурация" (the `bias` key: a bias on every
           Linear, the experts' included, on by default, off in Mixtral 8x7B)
           and the teaching-config table of "Подсчёт параметров" (each Linear
           gains d_out bias parameters): an expert with biases is
           (SiLU(u W_gate + b_gate) * (u W_up + b_up)) W_down + b_down.

Precision: fp32 by default, as the pages fix the router softmax in float32 and
the layer's oracle is stated in fp32; every function also runs in fp64 (pass
dtype=np.float64) for the error-bound pins.

Readings where the pages are silent (each listed in the design notes):
  * Top-k ties: larger logit first; exactly equal logits -> lower expert index.
  * Slot 0 holds the larger logit.
  * SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z}) (the pages defer SwiGLU to
    another chapter).
  * Combine weights stay in fp32 (no cast to the activation dtype).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# helpers: input widening (bf16 bit patterns -> float)
# ----------------------------------------------------------------------------
def widen(a: np.ndarray, dtype=np.float32) -> np.ndarray:
    """bf16 bit patterns (uint16) are widened exactly (bits << 16); floats are cast."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(dtype, copy=False)
    return a.astype(dtype, copy=False)


# ----------------------------------------------------------------------------
# router  [MIX-F], [MIX-IN]
# ----------------------------------------------------------------------------
def router_logits(x, w_gate, bias=None, dtype=np.float32) -> np.ndarray:
    """g = u W_r for every token row u ([MIX-F]); W_r stored [E, d] like nn.Linear.

    The optional per-expert bias is the Linear bias of the router ([MIX-IN]
    "Router: Linear(emb_size -> num_experts)").

    The pages fix the router's precision (fp32), not a summation order, so
    the fp32 logit is taken to be the fp32 value of the exact dot product:
    every product of a bf16 / fp32 input with an fp32 weight is exact in
    fp64, the sum is formed in fp64 and rounded once.  The bias is then added
    in fp32.
    """
    g = widen(x, np.float64) @ widen(w_gate, np.float64).T
    g = g.astype(dtype)
    if bias is not None:
        g = g + widen(bias, dtype)
    return g.astype(dtype, copy=False)


def top2(g: np.ndarray, k: int = 2) -> np.ndarray:
    """S = TopK(g, k) ([MIX-F]; Top2 keeps the two largest logits, [MIX-C]).

    Returns expert indices [T, k] int32, slot 0 = largest.  A stable sort of
    -g puts exactly equal logits in ascending expert order.
    """
    order = np.argsort(-g, axis=1, kind="stable")
    return np.ascontiguousarray(order[:, :k]).astype(np.int32)


def topk_softmax(g: np.ndarray, idx: np.ndarray, dtype=np.float32) -> np.ndarray:
    """w_i = e^{g_i} / sum_{j in S} e^{g_j} for i in S, computed in float32 ([MIX-F], [MIX-IN]).

    The max kept logit is subtracted first; it cancels in the ratio.
    """
    sel = np.take_along_axis(g.astype(dtype), idx.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    e = np.exp(sel - m)
    return (e / e.sum(axis=1, keepdims=True)).astype(dtype, copy=False)


def route_ref(x, w_gate, bias=None, k: int = 2, dtype=np.float32):
    """Router step: logits, top-k indices and combine weights."""
    g = router_logits(x, w_gate, bias, dtype)
    idx = top2(g, k)
    w = topk_softmax(g, idx, dtype)
    return g, idx, w


# ----------------------------------------------------------------------------
# expert  [MIX-F], [MIX-HF]
# ----------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + e^{-z})."""
    with np.errstate(over="ignore"):
        return z / (1 + np.exp(-z))


def expert_swiglu(u, w1_e, w3_e, w2_e, dtype=np.float32, b1_e=None, b3_e=None, b2_e=None) -> np.ndarray:
    """(SiLU(u W_gate) * (u W_up)) W_down for rows u ([MIX-F]); w1 = gate, w3 = up, w2 = down ([MIX-HF]).

    w1_e, w3_e are [d_ff, d] and w2_e is [d, d_ff] (nn.Linear layout).  The
    optional Linear biases b1_e, b3_e [d_ff] and b2_e [d] enter each
    projection's output ([MIX-B]); None means that Linear has no bias.
    """
    u = widen(u, dtype)
    a = u @ widen(w1_e, dtype).T
    if b1_e is not None:
        a = a + widen(b1_e, dtype)
    b = u @ widen(w3_e, dtype).T
    if b3_e is not None:
        b = b + widen(b3_e, dtype)
    h = silu(a) * b
    y = h @ widen(w2_e, dtype).T
    if b2_e is not None:
        y = y + widen(b2_e, dtype)
    return y.astype(dtype, copy=False)


def _expert_bias(eb, e):
    """(b1[e], b3[e], b2[e]) from eb = (b1 [E, d_ff] | None, b3 [E, d_ff] | None, b2 [E, d] | None)."""
    if eb is None:
        return None, None, None
    return tuple(None if b is None else b[e] for b in eb)


# ----------------------------------------------------------------------------
# O1: the definition, one token at a time  [MIX-F], [MIX-A] ("naive token loop")
# ----------------------------------------------------------------------------
def moe_forward_token_loop(x, w_gate, bias, w1, w3, w2, k: int = 2, dtype=np.float32, eb=None):
    """y_t = sum_{i in S_t} w_i SwiGLU_i(x_t), token by token.  Small inputs only.

    eb: optional expert biases (b1, b3, b2), see expert_swiglu."""
    g, idx, w = route_ref(x, w_gate, bias, k, dtype)
    X = widen(x, dtype)
    T, d = X.shape
    cache: Dict[int, Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}

    def weights(e):
        if e not in cache:
            cache[e] = (widen(w1[e], dtype), widen(w3[e], dtype), widen(w2[e], dtype))
        return cache[e]

    y = np.zeros((T, d), dtype=dtype)
    for t in range(T):
        acc = np.zeros(d, dtype=dtype)
        for s in range(k):
            e = int(idx[t, s])
            a, b, c = weights(e)
            acc = acc + w[t, s] * expert_swiglu(X[t:t + 1], a, b, c, dtype, *_expert_bias(eb, e))[0]
        y[t] = acc
    return y, (g, idx, w)


# ----------------------------------------------------------------------------
# O2: the pages' expert-major algorithm  [MIX-A]
# ----------------------------------------------------------------------------
def moe_forward_expert_loop(x, w_gate, bias, w1, w3, w2, k: int = 2, dtype=np.float32, eb=None):
    """Expert-major form ([MIX-A]): every expert runs once, on the block of
    tokens that selected it, and its outputs, scaled by the tokens' combine
    weights, are added into those tokens' rows of a zero output.

    The blocks are the dispatch permutation (dispatch_ref): expert e's block
    is rows offsets[e] .. offsets[e+1] of sorted_token, its tokens ascending;
    an empty block is not evaluated.  Row r of a block belongs to token
    sorted_token[r] and to the slot s with inv_pos[t, s] = r, whose weight
    scales it."""
    g, idx, w = route_ref(x, w_gate, bias, k, dtype)
    X = widen(x, dtype)
    T, d = X.shape
    E = widen(w_gate, dtype).shape[0]
    offsets, sorted_token, inv_pos = dispatch_ref(idx, E)
    rows = expert_rows_ref(X, sorted_token, offsets, w1, w3, w2, dtype, eb)
    slot_of_row = np.empty(T * k, dtype=np.int64)
    slot_of_row[inv_pos.reshape(-1)] = np.tile(np.arange(k), T)
    scale = w[sorted_token, slot_of_row].astype(dtype)
    Y = np.zeros((T, d), dtype=dtype)
    np.add.at(Y, sorted_token, scale[:, None] * rows)
    return Y, (g, idx, w)


def moe_forward_tokens(x_rows, w_gate, bias, w1, w3, w2, k: int = 2, dtype=np.float32, eb=None):
    """The layer on a subset of token rows.

    The MoE acts on each position independently (same page, exercise 6 of
    "Вопросы и упражнения"), so a sample of rows can be checked on its own.
    Uses the expert-major form; returns (y_rows, (g, idx, w)).
    """
    return moe_forward_expert_loop(x_rows, w_gate, bias, w1, w3, w2, k, dtype, eb)


# ----------------------------------------------------------------------------
# dispatch  [MIX-A]
# ----------------------------------------------------------------------------
def dispatch_ref(idx: np.ndarray, E: int):
    """Expert-sorted permutation in the order the pages' expert loop visits the
    (token, slot) pairs ([MIX-A]): expert by expert, each expert's tokens ascending.

    Returns (expert_offsets [E+1], sorted_token [T*k], inv_pos [T, k]):
    rows of expert e are sorted_token[offsets[e]:offsets[e+1]], tokens
    ascending; inv_pos[t, s] is the row that holds (token t, expert idx[t, s]).
    """
    T, k = idx.shape
    offsets = np.zeros(E + 1, dtype=np.int32)
    sorted_token = np.empty(T * k, dtype=np.int32)
    inv_pos = np.empty((T, k), dtype=np.int32)
    row = 0
    for e in range(E):
        offsets[e] = row
        tok, slot = np.nonzero(idx == e)
        for t, s in zip(tok.tolist(), slot.tolist()):
            sorted_token[row] = t
            inv_pos[t, s] = row
            row += 1
    offsets[E] = row
    return offsets, sorted_token, inv_pos


def combine_ref(y_sorted, inv_pos, topk_w, residual=None, dtype=np.float32) -> np.ndarray:
    """Y[t] = sum_s w[t, s] * Expert_{idx[t,s]}(x_t), read back from the expert-sorted rows.

    The index-add of [MIX-A] written as a gather: row inv_pos[t, s] of
    y_sorted holds the output of token t's slot-s expert.  Slots are added in
    order, starting from zero (or from the residual row when given).
    """
    T, k = inv_pos.shape
    out = np.zeros((T, y_sorted.shape[1]), dtype=dtype)
    for s in range(k):
        out = out + topk_w[:, s:s + 1].astype(dtype) * y_sorted[inv_pos[:, s]].astype(dtype)
    if residual is not None:
        out = out + widen(residual, dtype)
    return out


def expert_rows_ref(x, sorted_token, offsets, w1, w3, w2, dtype=np.float32, eb=None) -> np.ndarray:
    """y_sorted[r] = Expert_e(x[sorted_token[r]]) for the rows of every expert e ([MIX-A], [MIX-F])."""
    E = len(offsets) - 1
    X = widen(x, dtype)
    d = X.shape[1]
    out = np.zeros((int(offsets[-1]), d), dtype=dtype)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = expert_swiglu(X[sorted_token[lo:hi]], w1[e], w3[e], w2[e], dtype, *_expert_bias(eb, e))
    return out


# ----------------------------------------------------------------------------
# RMSNorm and the residual MoE sublayer  [MIX-F]
# ----------------------------------------------------------------------------
def rmsnorm_ref(z, gamma=None, eps: float = 1e-5, dtype=np.float32) -> np.ndarray:
    """RMSNorm(z) = z / sqrt(mean_j z_j^2 + eps) * gamma, row by row ([MIX-F])."""
    z = widen(z, dtype)
    r = np.sqrt(np.mean(z * z, axis=1, keepdims=True) + dtype(eps))
    out = z / r
    if gamma is not None:
        out = out * widen(gamma, dtype)
    return out.astype(dtype, copy=False)


def block_forward_ref(h, gamma, eps, w_gate, bias, w1, w3, w2, k: int = 2, dtype=np.float32, eb=None):
    """H = U + MoE(RMSNorm_2(U)) ([MIX-F], pre-LN block, MoE half).

    Returns (h_out, u, (g, idx, w)) with u the normalised input of the MoE.
    """
    U = widen(h, dtype)
    u = rmsnorm_ref(U, gamma, eps, dtype)
    y, route = moe_forward_expert_loop(u, w_gate, bias, w1, w3, w2, k, dtype, eb)
    return (U + y).astype(dtype, copy=False), u, route


# ----------------------------------------------------------------------------
# load-balancing loss  [MIX-LB]
# ----------------------------------------------------------------------------
def router_stats_ref(logits_per_layer: Sequence[np.ndarray], E: int, k: int,
                     token_mask: Optional[np.ndarray] = None, dtype=np.float64):
    """f [k, E] and P [E] of the load-balancing loss ([MIX-LB]).

    f_{s,i}: share of tokens whose slot-s expert (s-th largest logit, the
    top-k order) is i; P_i: mean over tokens of the router's softmax over all
    E experts.  The statistics pool every MoE layer and every unmasked token.
    """
    g_all: List[np.ndarray] = []
    for g in logits_per_layer:
        g = np.asarray(g, dtype=dtype)
        if token_mask is not None:
            g = g[np.asarray(token_mask, dtype=bool)]
        g_all.append(g)
    G = np.concatenate(g_all, axis=0)
    n = G.shape[0]
    f = np.zeros((k, E), dtype=dtype)
    P = np.zeros(E, dtype=dtype)
    if n == 0:
        return f, P
    idx = top2(G, k)
    for s in range(k):
        for i in range(E):
            f[s, i] = np.count_nonzero(idx[:, s] == i) / n
    ex = np.exp(G - G.max(axis=1, keepdims=True))
    probs = ex / ex.sum(axis=1, keepdims=True)
    P = probs.mean(axis=0)
    return f, P


def aux_loss_ref(logits_per_layer: Sequence[np.ndarray], E: int, k: int, alpha: float = 1.0,
                 token_mask: Optional[np.ndarray] = None, dtype=np.float64) -> float:
    """alpha * E * sum_{s=1..k} sum_i f_{s,i} P_i over all layers' real tokens ([MIX-LB])."""
    f, P = router_stats_ref(logits_per_layer, E, k, token_mask, dtype)
    return float(alpha * E * np.sum(f * P[None, :]))
