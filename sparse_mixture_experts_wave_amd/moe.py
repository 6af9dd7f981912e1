"""Python binding of the MoE C ABI: same entry points, torch tensors in and out.

Argument marshalling only.  torch allocates device memory and supplies the
current HIP stream; every step of the layer runs in the HIP kernels of
libmoe.so.  Tensors must be contiguous and on the GPU; bf16 data is passed
as torch.bfloat16 (its bits are what the kernels read).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib

_DT = {torch.float32: _lib.MOE_F32, torch.bfloat16: _lib.MOE_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")
    return _DT[t.dtype]


def _gpu(t: Optional[torch.Tensor], name: str) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def make_shape(T: int, d: int, d_ff: int, E: int, k: int = 2,
               act: torch.dtype = torch.bfloat16, wt: Optional[torch.dtype] = None) -> _lib.MoEShape:
    wt = act if wt is None else wt
    return _lib.MoEShape(int(T), int(d), int(d_ff), int(E), int(k), _DT.get(act, -1), _DT.get(wt, -1))


def workspace_size(shape: _lib.MoEShape) -> int:
    return int(_lib.load().moe_workspace_size(ctypes.byref(shape)))


def expert_ffn_workspace_size(shape: _lib.MoEShape) -> int:
    return int(_lib.load().moe_expert_ffn_workspace_size(ctypes.byref(shape)))


def _expert_bias(b1: Optional[torch.Tensor], b3: Optional[torch.Tensor], b2: Optional[torch.Tensor],
                 E: int, d: int, d_ff: int, wt: torch.dtype):
    """Pointer to a moe_expert_bias struct, or None when no bias is given."""
    if b1 is None and b3 is None and b2 is None:
        return None
    for t, name, n in ((b1, "b1", d_ff), (b3, "b3", d_ff), (b2, "b2", d)):
        if t is not None:
            _gpu(t, name)
            if t.dtype != wt or tuple(t.shape) != (E, n):
                raise ValueError(f"{name} must be [{E}, {n}] in the weight dtype {wt}")
    return ctypes.byref(_lib.MoEExpertBias(_p(b1), _p(b3), _p(b2)))


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# The C ABI sees only pointers: the layouts include/moe.h states are checked
# here, so that a mis-shaped or mis-typed tensor raises instead of being read
# or written past its end.
def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} {list(shape)}, got {t.dtype} {list(t.shape)}")


def _rows(t: torch.Tensor, name: str, dtype: torch.dtype, rows: int, cols: Optional[int] = None) -> None:
    """t must hold at least `rows` rows (of `cols` columns when given) of dtype."""
    ok = t.dtype == dtype and t.dim() == (1 if cols is None else 2) and t.shape[0] >= rows
    if ok and cols is not None:
        ok = t.shape[1] == cols
    if not ok:
        want = f"[>= {rows}]" if cols is None else f"[>= {rows}, {cols}]"
        raise ValueError(f"{name} must be {dtype} {want}, got {t.dtype} {list(t.shape)}")


def _activations(x: torch.Tensor, name: str = "x"):
    if x.dim() != 2:
        raise ValueError(f"{name} must be [T, d], got {list(x.shape)}")
    return x.shape


def _layer_weights(d: int, w_gate: Optional[torch.Tensor], bias: Optional[torch.Tensor], w1: torch.Tensor,
                   w3: torch.Tensor, w2: torch.Tensor):
    """Router (fp32 [E, d], bias fp32 [E]) and expert weights (w1, w3 [E, d_ff, d], w2 [E, d, d_ff], one
    dtype) against the activation width d -> (E, d_ff)."""
    if w1.dim() != 3:
        raise ValueError(f"w1 must be [E, d_ff, d], got {list(w1.shape)}")
    E, d_ff, _ = w1.shape
    _need(w1, "w1", w1.dtype, (E, d_ff, d))
    _need(w3, "w3", w1.dtype, (E, d_ff, d))
    _need(w2, "w2", w1.dtype, (E, d, d_ff))
    if w_gate is not None:
        _need(w_gate, "w_gate", torch.float32, (E, d))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    return E, d_ff


# d_ff does not enter the router, dispatch or combine; any valid value does.
_D_FF_UNUSED = 64


def moe_route(x: torch.Tensor, w_gate: torch.Tensor, bias: Optional[torch.Tensor] = None, k: int = 2,
              want_logits: bool = False) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Router logits -> (topk_idx [T,k] int32, topk_w [T,k] fp32, logits [T,E] fp32 or None)."""
    x, w_gate, bias = _gpu(x, "x"), _gpu(w_gate, "w_gate"), _gpu(bias, "bias")
    T, d = _activations(x)
    E = w_gate.shape[0]
    _need(w_gate, "w_gate", torch.float32, (E, d))
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    shape = make_shape(T, d, _D_FF_UNUSED, E, k, x.dtype)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if want_logits else None
    _lib.check(_lib.load().moe_route(ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(logits), _p(idx),
                                     _p(w), _stream(x)))
    return idx, w, logits


def moe_dispatch(topk_idx: torch.Tensor, E: int, d: int = 64):
    """-> (expert_offsets [E+1], sorted_token [T*k], inv_pos [T,k]) int32."""
    topk_idx = _gpu(topk_idx, "topk_idx")
    if topk_idx.dtype != torch.int32 or topk_idx.dim() != 2:
        raise ValueError(f"topk_idx must be int32 [T, k], got {topk_idx.dtype} {list(topk_idx.shape)}")
    T, k = topk_idx.shape
    shape = make_shape(T, d, _D_FF_UNUSED, E, k, torch.bfloat16)
    dev = topk_idx.device
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    st = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    inv = torch.empty((T, k), dtype=torch.int32, device=dev)
    _lib.check(_lib.load().moe_dispatch(ctypes.byref(shape), _p(topk_idx), _p(off), _p(st), _p(inv), None, 0,
                                        _stream(topk_idx)))
    return off, st[:T * k], inv


def moe_expert_ffn(x: torch.Tensor, expert_offsets: torch.Tensor, sorted_token: torch.Tensor,
                   w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor, k: int = 2,
                   y_sorted: Optional[torch.Tensor] = None, b1: Optional[torch.Tensor] = None,
                   b3: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Expert SwiGLU on every dispatched row -> y_sorted [T*k, d] fp32.

    b1, b3 [E, d_ff] and b2 [E, d] are the experts' optional Linear biases."""
    x, w1, w3, w2 = _gpu(x, "x"), _gpu(w1, "w1"), _gpu(w3, "w3"), _gpu(w2, "w2")
    expert_offsets, sorted_token = _gpu(expert_offsets, "expert_offsets"), _gpu(sorted_token, "sorted_token")
    T, d = _activations(x)
    E, d_ff = _layer_weights(d, None, None, w1, w3, w2)
    _need(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    _rows(sorted_token, "sorted_token", torch.int32, T * k)
    shape = make_shape(T, d, d_ff, E, k, x.dtype, w1.dtype)
    if y_sorted is None:
        y_sorted = torch.empty((max(T * k, 1), d), dtype=torch.float32, device=x.device)
    _rows(_gpu(y_sorted, "y_sorted"), "y_sorted", torch.float32, T * k, d)
    ws = _ws(expert_ffn_workspace_size(shape), x.device)
    eb = _expert_bias(b1, b3, b2, E, d, d_ff, w1.dtype)
    _lib.check(_lib.load().moe_expert_ffn(ctypes.byref(shape), _p(x), _p(expert_offsets), _p(sorted_token),
                                          _p(w1), _p(w3), _p(w2), eb, _p(y_sorted), _p(ws), ws.numel(),
                                          _stream(x)))
    return y_sorted[:T * k]


def moe_combine(y_sorted: torch.Tensor, inv_pos: torch.Tensor, topk_w: torch.Tensor, E: int,
                out_dtype: torch.dtype = torch.bfloat16, residual: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[t] = sum_s w[t,s] * y_sorted[inv_pos[t,s]] (+ residual[t]) -> [T, d] in out_dtype."""
    y_sorted, inv_pos, topk_w = _gpu(y_sorted, "y_sorted"), _gpu(inv_pos, "inv_pos"), _gpu(topk_w, "topk_w")
    residual = _gpu(residual, "residual")
    if inv_pos.dim() != 2 or y_sorted.dim() != 2:
        raise ValueError("inv_pos must be [T, k] and y_sorted [rows, d]")
    T, k = inv_pos.shape
    d = y_sorted.shape[1]
    _need(inv_pos, "inv_pos", torch.int32, (T, k))
    _need(topk_w, "topk_w", torch.float32, (T, k))
    _rows(y_sorted, "y_sorted", torch.float32, T * k, d)
    if residual is not None:
        _need(residual, "residual", out_dtype, (T, d))
    shape = make_shape(T, d, _D_FF_UNUSED, E, k, out_dtype)
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=y_sorted.device)
    _need(_gpu(out, "out"), "out", out_dtype, (T, d))
    _lib.check(_lib.load().moe_combine(ctypes.byref(shape), _p(y_sorted), _p(inv_pos), _p(topk_w), _p(residual),
                                       _p(out), _stream(y_sorted)))
    return out


def moe_forward(x: torch.Tensor, w_gate: torch.Tensor, bias: Optional[torch.Tensor], w1: torch.Tensor,
                w3: torch.Tensor, w2: torch.Tensor, k: int = 2, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, b1: Optional[torch.Tensor] = None,
                b3: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole layer y = sum_{i in Top2} softmax_i * SwiGLU_i(x) -> [T, d] in x.dtype.

    bias is the router's; b1, b3 [E, d_ff] and b2 [E, d] the experts' optional Linear biases."""
    x, w_gate, bias = _gpu(x, "x"), _gpu(w_gate, "w_gate"), _gpu(bias, "bias")
    w1, w3, w2 = _gpu(w1, "w1"), _gpu(w3, "w3"), _gpu(w2, "w2")
    T, d = _activations(x)
    E, d_ff = _layer_weights(d, w_gate, bias, w1, w3, w2)
    shape = make_shape(T, d, d_ff, E, k, x.dtype, w1.dtype)
    if out is None:
        out = torch.empty_like(x)
    _need(_gpu(out, "out"), "out", x.dtype, (T, d))
    if workspace is None:
        workspace = _ws(workspace_size(shape), x.device)
    eb = _expert_bias(b1, b3, b2, E, d, d_ff, w1.dtype)
    _lib.check(_lib.load().moe_forward(ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2),
                                       eb, _p(out), _p(workspace), workspace.numel(), _stream(x)))
    return out


def moe_forward_noalloc(x: torch.Tensor, w_gate: torch.Tensor, bias: Optional[torch.Tensor], w1: torch.Tensor,
                        w3: torch.Tensor, w2: torch.Tensor, k: int = 2, out: Optional[torch.Tensor] = None,
                        b1: Optional[torch.Tensor] = None, b3: Optional[torch.Tensor] = None,
                        b2: Optional[torch.Tensor] = None) -> torch.Tensor:
    """moe_forward without a workspace: the library's static per-GPU scratch holds
    the intermediates.  Nothing is allocated when out is given."""
    x, w_gate, bias = _gpu(x, "x"), _gpu(w_gate, "w_gate"), _gpu(bias, "bias")
    w1, w3, w2 = _gpu(w1, "w1"), _gpu(w3, "w3"), _gpu(w2, "w2")
    T, d = _activations(x)
    E, d_ff = _layer_weights(d, w_gate, bias, w1, w3, w2)
    shape = make_shape(T, d, d_ff, E, k, x.dtype, w1.dtype)
    if out is None:
        out = torch.empty_like(x)
    _need(_gpu(out, "out"), "out", x.dtype, (T, d))
    eb = _expert_bias(b1, b3, b2, E, d, d_ff, w1.dtype)
    _lib.check(_lib.load().moe_forward_noalloc(ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3),
                                               _p(w2), eb, _p(out), _stream(x)))
    return out


def moe_block_forward(h: torch.Tensor, gamma: torch.Tensor, eps: float, w_gate: torch.Tensor,
                      bias: Optional[torch.Tensor], w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor,
                      k: int = 2, workspace: Optional[torch.Tensor] = None, b1: Optional[torch.Tensor] = None,
                      b3: Optional[torch.Tensor] = None, b2: Optional[torch.Tensor] = None) -> torch.Tensor:
    """In place: h <- h + MoE(RMSNorm(h) * gamma).  Returns h."""
    h, gamma, w_gate, bias = _gpu(h, "h"), _gpu(gamma, "gamma"), _gpu(w_gate, "w_gate"), _gpu(bias, "bias")
    w1, w3, w2 = _gpu(w1, "w1"), _gpu(w3, "w3"), _gpu(w2, "w2")
    T, d = _activations(h, "h")
    E, d_ff = _layer_weights(d, w_gate, bias, w1, w3, w2)
    _need(gamma, "gamma", torch.float32, (d,))
    shape = make_shape(T, d, d_ff, E, k, h.dtype, w1.dtype)
    if workspace is None:
        workspace = _ws(workspace_size(shape), h.device)
    eb = _expert_bias(b1, b3, b2, E, d, d_ff, w1.dtype)
    _lib.check(_lib.load().moe_block_forward(ctypes.byref(shape), _p(h), _p(gamma), float(eps), _p(w_gate),
                                             _p(bias), _p(w1), _p(w3), _p(w2), eb, _p(workspace),
                                             workspace.numel(), _stream(h)))
    return h


def moe_aux_loss(logits: torch.Tensor, k: int = 2, alpha: float = 1.0,
                 token_mask: Optional[torch.Tensor] = None, want_stats: bool = False):
    """Load-balancing loss over router logits [L, T, E] (or [T, E]) -> (loss [1], stats or None).

    stats is [(k+1)*E]: f_{s,i} at s*E + i, then P_i at k*E + i."""
    logits = _gpu(logits, "logits")
    if logits.dtype != torch.float32:
        raise ValueError("logits must be float32")
    if logits.dim() == 2:
        logits = logits.unsqueeze(0)
    L, T, E = logits.shape
    if token_mask is not None:
        token_mask = _gpu(token_mask, "token_mask")
        if token_mask.dtype not in (torch.uint8, torch.bool) or token_mask.numel() != T:
            raise ValueError("token_mask must be uint8/bool [T]")
        token_mask = token_mask.to(torch.uint8)
    shape = make_shape(T, 64, _D_FF_UNUSED, E, k, torch.bfloat16)
    loss = torch.empty(1, dtype=torch.float32, device=logits.device)
    stats = torch.empty((k + 1) * E, dtype=torch.float32, device=logits.device) if want_stats else None
    _lib.check(_lib.load().moe_aux_loss(ctypes.byref(shape), _p(logits), int(L), _p(token_mask), float(alpha),
                                        _p(loss), _p(stats), _stream(logits)))
    return loss, stats


# ---------------------------------------------------------------------------
# the attention sublayer around the MoE
# ---------------------------------------------------------------------------
def make_attn_shape(T: int, d: int, H: int, G: int, d_h: int, act: torch.dtype = torch.bfloat16) -> _lib.MoEAttnShape:
    return _lib.MoEAttnShape(int(T), int(d), int(H), int(G), int(d_h), _DT.get(act, -1))


def attention_workspace_size(shape: _lib.MoEAttnShape) -> int:
    return int(_lib.load().moe_attention_workspace_size(ctypes.byref(shape)))


def moe_gqa_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, d: Optional[int] = None,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal GQA attention on rotated heads: q [T, H, d_h], k, v [T, G, d_h] -> o [T, H, d_h]."""
    q, k, v = _gpu(q, "q"), _gpu(k, "k"), _gpu(v, "v")
    T, H, dh = q.shape
    G = k.shape[1]
    if tuple(k.shape) != (T, G, dh) or tuple(v.shape) != (T, G, dh):
        raise ValueError("k and v must be [T, G, d_h] with q [T, H, d_h]")
    if v.dtype != q.dtype or k.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    shape = make_attn_shape(T, d if d is not None else H * dh, H, G, dh, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    _need(_gpu(out, "out"), "out", q.dtype, (T, H, dh))
    _lib.check(_lib.load().moe_gqa_attention(ctypes.byref(shape), _p(q), _p(k), _p(v), _p(out), _stream(q)))
    return out


def moe_attention_block_forward(h: torch.Tensor, gamma: torch.Tensor, eps: float, wqkv: torch.Tensor,
                                wo: torch.Tensor, H: int, G: int, rope_theta: float = 1e6, pos0: int = 0,
                                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """In place: h <- h + GQA(RMSNorm(h) * gamma) with RoPE (causal, positions pos0 ..).

    wqkv is [(H + 2G) d_h, d]: W_Q rows, then W_K, then W_V; wo is [d, H d_h]."""
    h, gamma, wqkv, wo = _gpu(h, "h"), _gpu(gamma, "gamma"), _gpu(wqkv, "wqkv"), _gpu(wo, "wo")
    T, d = _activations(h, "h")
    if wo.dim() != 2 or H < 1 or wo.shape[1] % H != 0:
        raise ValueError(f"wo must be [d, H d_h], got {list(wo.shape)} with H = {H}")
    dh = wo.shape[1] // H
    _need(wqkv, "wqkv", h.dtype, ((H + 2 * G) * dh, d))
    _need(wo, "wo", h.dtype, (d, H * dh))
    _need(gamma, "gamma", torch.float32, (d,))
    shape = make_attn_shape(T, d, H, G, dh, h.dtype)
    if workspace is None:
        workspace = _ws(attention_workspace_size(shape), h.device)
    _lib.check(_lib.load().moe_attention_block_forward(ctypes.byref(shape), _p(h), _p(gamma), float(eps), _p(wqkv),
                                                       _p(wo), float(rope_theta), int(pos0), _p(workspace),
                                                       workspace.numel(), _stream(h)))
    return h
