"""Seeded input generator for the Mixtral sparse MoE feed-forward layer.

The workloads follow the layer shapes of Mixtral 8x7B (d = 4096, d_ff = 14336,
E = 8 experts, top-2), as listed on the "Mixtral" textbook page, section
"Научный вклад" (architecture bullet), plus a tiny fp32 case.

Distributions.  "N(0, s)" with s a number means standard deviation s (the
textbook's initialiser, "Разбор кода" / Mixtral __init__, draws Linear weights
with std 0.02).  "N(0, 1/fan_in)" means variance 1/fan_in.  Every tensor has its
own numpy stream seeded by SeedSequence(seed, spawn_key=(config id, layer,
tensor id)); matrices are drawn in row-major storage order.

Storage layout (nn.Linear convention, reduction dimension contiguous):
  x      [T, d]            activations
  w_gate [E, d]   fp32     router
  bias   [E]      fp32     router bias or None
  w1     [E, d_ff, d]      gate projection  (HF name w1)
  w3     [E, d_ff, d]      up projection    (HF name w3)
  w2     [E, d, d_ff]      down projection  (HF name w2)
  b1, b3 [E, d_ff], b2 [E, d]   optional expert Linear biases (weight dtype),
         drawn N(0, expert_bias_std) when that is nonzero, else None
bf16 tensors are returned as uint16 bit patterns, rounded from fp32 to
nearest-even.  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

TENSOR_IDS = {"x": 0, "w_gate": 1, "w1": 2, "w3": 3, "w2": 4, "b1": 6, "b3": 7, "b2": 8}


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int
    T: int
    d: int
    d_ff: int
    E: int = 8
    k: int = 2
    dtype: str = "bf16"            # "f32" or "bf16": activations and expert weights
    x_unit_rms: bool = False       # rows of x scaled onto the sphere of radius sqrt(d)
    wg_std: float = 0.02           # std of the router weights
    bias: Optional[str] = None     # None or "zipf1.2"
    expert_bias_std: float = 0.0   # 0: experts without Linear biases (Mixtral 8x7B)
    layers: int = 1
    description: str = ""

    @property
    def w1_std(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def w2_std(self) -> float:
        return 1.0 / math.sqrt(self.d_ff)

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


_MIXTRAL = dict(d=4096, d_ff=14336, E=8, k=2)

CONFIGS: Dict[str, MoEConfig] = {
    c.name: c
    for c in [
        MoEConfig("tiny_fp32", 0, T=64, d=128, d_ff=256, dtype="f32", wg_std=0.02,
                  description="tiny MoE layer, fp32, T=64 d=128 d_ff=256 E=8 k=2"),
        MoEConfig("mixtral_decode_t16", 1, T=16, dtype="bf16", x_unit_rms=True,
                  wg_std=1.0 / math.sqrt(4096), **_MIXTRAL,
                  description="Mixtral 8x7B MoE layer, decode regime, T=16, bf16"),
        MoEConfig("mixtral_prefill_t4096", 2, T=4096, dtype="bf16", wg_std=0.02, **_MIXTRAL,
                  description="Mixtral 8x7B MoE layer, prefill regime, T=4096, bf16"),
        MoEConfig("mixtral_skewed_t16384", 3, T=16384, dtype="bf16", wg_std=0.02,
                  bias="zipf1.2", **_MIXTRAL,
                  description="Mixtral 8x7B MoE layer, Zipf(1.2) router bias, T=16384, bf16"),
        MoEConfig("mixtral_stack32_t2048", 4, T=2048, dtype="bf16", wg_std=0.02, layers=32,
                  **_MIXTRAL,
                  description="32 pre-RMSNorm residual MoE sublayers, T=2048, bf16"),
    ]
}


def config_by_name(name: str) -> MoEConfig:
    return CONFIGS[name]


def zipf_router_bias(E: int, s: float = 1.2) -> np.ndarray:
    """Router bias b_e = ln p_e with p_e proportional to (e+1)^-s: expert 0 heaviest."""
    p = np.array([(e + 1.0) ** (-s) for e in range(E)], dtype=np.float64)
    p /= p.sum()
    return np.log(p).astype(np.float32)


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF))) >> 16
    return r.astype(np.uint16)


def _rng(seed: int, cfg: MoEConfig, layer: int, tensor: str) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(cfg.cfg_id, layer, TENSOR_IDS[tensor]))
    return np.random.default_rng(ss)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f32(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def _expert_stack(rng, E, rows, cols, std, dtype):
    out = np.empty((E, rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for e in range(E):  # one expert at a time keeps the fp32 staging small
        out[e] = _store(_normal(rng, (rows, cols), std), dtype)
    return out


def _unit_rms_rows(z: np.ndarray) -> np.ndarray:
    """Scale each row onto the sphere of radius sqrt(len(row)) (input recipe only)."""
    z64 = z.astype(np.float64)
    scale = np.sqrt(np.mean(z64 * z64, axis=1, keepdims=True))
    return (z64 / scale).astype(np.float32)


def generate(cfg: MoEConfig, layer: int = 0, seed: int = 0,
             tensors=("x", "w_gate", "w1", "w3", "w2")) -> Dict[str, Optional[np.ndarray]]:
    """Draw the named tensors of one layer of `cfg` on the host with numpy."""
    out: Dict[str, Optional[np.ndarray]] = {}
    if "x" in tensors:
        x = _normal(_rng(seed, cfg, layer, "x"), (cfg.T, cfg.d), 1.0)
        if cfg.x_unit_rms:
            x = _unit_rms_rows(x)
        out["x"] = _store(x, cfg.dtype)
    if "w_gate" in tensors:
        out["w_gate"] = _normal(_rng(seed, cfg, layer, "w_gate"), (cfg.E, cfg.d), cfg.wg_std)
    out["bias"] = zipf_router_bias(cfg.E) if cfg.bias == "zipf1.2" else None
    if "w1" in tensors:
        out["w1"] = _expert_stack(_rng(seed, cfg, layer, "w1"), cfg.E, cfg.d_ff, cfg.d, cfg.w1_std, cfg.dtype)
    if "w3" in tensors:
        out["w3"] = _expert_stack(_rng(seed, cfg, layer, "w3"), cfg.E, cfg.d_ff, cfg.d, cfg.w1_std, cfg.dtype)
    if "w2" in tensors:
        out["w2"] = _expert_stack(_rng(seed, cfg, layer, "w2"), cfg.E, cfg.d, cfg.d_ff, cfg.w2_std, cfg.dtype)
    for name, cols in (("b1", cfg.d_ff), ("b3", cfg.d_ff), ("b2", cfg.d)):
        out[name] = (_store(_normal(_rng(seed, cfg, layer, name), (cfg.E, cols), cfg.expert_bias_std), cfg.dtype)
                     if cfg.expert_bias_std > 0 else None)
    return out


def _torch_seed(seed: int, cfg: MoEConfig, layer: int, tensor: str) -> int:
    ss = np.random.SeedSequence(seed, spawn_key=(cfg.cfg_id, layer, TENSOR_IDS[tensor], 0x7041))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def generate_torch(cfg: MoEConfig, device, layer: int = 0, seed: int = 0):
    """Draw one layer of `cfg` directly in device memory with torch's seeded generator.

    Same distributions and layout as `generate`, different streams (torch's
    Philox instead of numpy's PCG64), so it is fast at Mixtral sizes.  bf16
    tensors are torch.bfloat16 (fp32 draw, rounded to nearest-even).
    """
    import torch

    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def normal(shape, std, tensor):
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(seed, cfg, layer, tensor))
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(std)

    def stack(rows, cols, std, tensor):
        g = torch.Generator(device=device)
        g.manual_seed(_torch_seed(seed, cfg, layer, tensor))
        out = torch.empty((cfg.E, rows, cols), device=device, dtype=dt)
        for e in range(cfg.E):
            out[e].copy_(torch.randn((rows, cols), generator=g, device=device,
                                     dtype=torch.float32).mul_(std))
        return out

    x = normal((cfg.T, cfg.d), 1.0, "x")
    if cfg.x_unit_rms:
        x = (x.double() / x.double().pow(2).mean(dim=1, keepdim=True).sqrt()).float()
    res = {
        "x": x.to(dt).contiguous(),
        "w_gate": normal((cfg.E, cfg.d), cfg.wg_std, "w_gate").contiguous(),
        "bias": (torch.from_numpy(zipf_router_bias(cfg.E)).to(device)
                 if cfg.bias == "zipf1.2" else None),
        "w1": stack(cfg.d_ff, cfg.d, cfg.w1_std, "w1"),
        "w3": stack(cfg.d_ff, cfg.d, cfg.w1_std, "w3"),
        "w2": stack(cfg.d, cfg.d_ff, cfg.w2_std, "w2"),
    }
    return res


# ---------------------------------------------------------------------------
# inputs of the attention sublayer around the MoE (GQA with RoPE)
# ---------------------------------------------------------------------------
ATTN_TENSOR_IDS = {"h": 20, "wqkv": 21, "wo": 22, "q": 23, "k": 24, "v": 25, "gamma": 26}


def _attn_rng(seed: int, cfg_id: int, tensor: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(cfg_id, 0, ATTN_TENSOR_IDS[tensor])))


def attention_inputs(T: int, d: int, H: int, G: int, dh: int, cfg_id: int = 40, seed: int = 0,
                     gamma: str = "ones") -> Dict[str, np.ndarray]:
    """One sublayer's inputs, bf16 bits: h [T, d] ~ N(0, 1); wqkv [(H + 2G) dh, d] and
    wo [d, H dh] with variance 1/fan_in (rows of W_Q, then W_K, then W_V); gamma fp32
    ones (the pages' initial value) or uniform(0.5, 1.5) with gamma="random"."""
    out = {
        "h": bf16_bits_from_f32(_normal(_attn_rng(seed, cfg_id, "h"), (T, d), 1.0)),
        "wqkv": bf16_bits_from_f32(_normal(_attn_rng(seed, cfg_id, "wqkv"), ((H + 2 * G) * dh, d), 1 / math.sqrt(d))),
        "wo": bf16_bits_from_f32(_normal(_attn_rng(seed, cfg_id, "wo"), (d, H * dh), 1 / math.sqrt(H * dh))),
    }
    if gamma == "ones":
        out["gamma"] = np.ones(d, np.float32)
    else:
        out["gamma"] = _attn_rng(seed, cfg_id, "gamma").uniform(0.5, 1.5, d).astype(np.float32)
    return out


def attention_heads(T: int, H: int, G: int, dh: int, cfg_id: int = 41, seed: int = 0) -> Dict[str, np.ndarray]:
    """Rotated-head inputs of the attention core, bf16 bits: q [T, H, dh], k, v [T, G, dh] ~ N(0, 1)."""
    return {n: bf16_bits_from_f32(_normal(_attn_rng(seed, cfg_id, n), (T, H if n == "q" else G, dh), 1.0))
            for n in ("q", "k", "v")}
