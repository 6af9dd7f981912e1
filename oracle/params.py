"""Analytic parameter counts of the models on the pages.

TEST INFRASTRUCTURE ONLY.

Formulas: "Mixtral" textbook page, section "Подсчёт параметров" (parameter
count): N_attn = d*H*d_h + 2*d*G*d_h + H*d_h*d, N_exp = 3*d*d_ff,
N_total = V*d + L*(N_attn + d*E + E*N_exp + 2d) + d + d*V, and N_active with
k experts in place of E.  With bias every Linear also gets d_out parameters
(the teaching-config table on the same page).  The dense Mistral count is the
same sum with one SwiGLU FFN per layer ("Mistral" textbook page, parameter
count section).
"""
from __future__ import annotations


def _linear(d_in: int, d_out: int, bias: bool) -> int:
    return d_in * d_out + (d_out if bias else 0)


def moe_model_param_counts(d: int, L: int, H: int, G: int, d_h: int, d_ff: int, E: int, k: int,
                           V: int, bias: bool = False) -> dict:
    """Per-part and total counts of a Mixtral-style model (untied output head)."""
    attn = (_linear(d, H * d_h, bias) + 2 * _linear(d, G * d_h, bias) + _linear(H * d_h, d, bias))
    router = _linear(d, E, bias)
    expert = 2 * _linear(d, d_ff, bias) + _linear(d_ff, d, bias)
    norms = 2 * d
    layer = attn + router + E * expert + norms
    emb_out = V * d + _linear(d, V, bias)
    total = L * layer + emb_out + d
    active = total - L * (E - k) * expert
    return {
        "attention_layer": attn,
        "router_layer": router,
        "expert": expert,
        "experts_layer": E * expert,
        "norms_layer": norms,
        "layer": layer,
        "layers": L * layer,
        "emb_out": emb_out,
        "experts_all": L * E * expert,
        "total": total,
        "active": active,
    }


def mistral_param_count(d: int, L: int, H: int, G: int, d_h: int, d_ff: int, V: int,
                        bias: bool = False) -> int:
    """Dense Mistral: one SwiGLU FFN (3*d*d_ff, plus biases) per layer in place of the MoE."""
    attn = (_linear(d, H * d_h, bias) + 2 * _linear(d, G * d_h, bias) + _linear(H * d_h, d, bias))
    ffn = 2 * _linear(d, d_ff, bias) + _linear(d_ff, d, bias)
    return V * d + L * (attn + ffn + 2 * d) + d + _linear(d, V, bias)
