"""CPU oracle for the Mixtral sparse MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
anything under this directory: only the tests, the smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP library; the
one module both sides use is the seeded input generator in ``synth``.

Every function restates, in plain numpy, a passage of the pages it cites
(page title + section / equation).  Results the pages fix (parameter counts,
closed forms, invariants) pin it in ``tests/test_oracle_pins.py``.

Every function is pinned to something other than itself: the whole layer
(both its token-loop and expert-loop forms) to HuggingFace's
MixtralSparseMoeBlock in float64, the load-balancing loss to HF's
load_balancing_loss_func, RoPE and the GQA attention to HF's
MixtralRotaryEmbedding / MixtralAttention after the pages' q/k row
permutation, plus the invariants and brute-force cases listed in the pin
tests (identity case, 28-pair brute force, fp64 shadow, parameter counts).
"""
from .moe_ref import (  # noqa: F401
    aux_loss_ref,
    block_forward_ref,
    combine_ref,
    dispatch_ref,
    expert_rows_ref,
    expert_swiglu,
    moe_forward_expert_loop,
    moe_forward_token_loop,
    moe_forward_tokens,
    rmsnorm_ref,
    route_ref,
    router_stats_ref,
    router_logits,
    silu,
    top2,
    topk_softmax,
    widen,
)
from .attn_ref import attention_sublayer_ref, gqa_attention_ref, rope_ref  # noqa: F401
from .params import mistral_param_count, moe_model_param_counts  # noqa: F401
