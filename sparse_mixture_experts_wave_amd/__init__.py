"""MI355X (gfx950) Mixtral sparse MoE feed-forward layer.

y = sum_{i in Top2(x W_g)} softmax_i * (SiLU(x W1_i) * (x W3_i)) W2_i, computed by
hand-written HIP kernels behind the C ABI in include/moe.h (libmoe.so), and the
GQA + RoPE attention sublayer around it.
"""
from ._lib import LIB_PATH, MoEError, load  # noqa: F401
from .moe import (  # noqa: F401
    attention_workspace_size,
    expert_ffn_workspace_size,
    make_attn_shape,
    moe_attention_block_forward,
    moe_gqa_attention,
    make_shape,
    moe_aux_loss,
    moe_block_forward,
    moe_combine,
    moe_dispatch,
    moe_expert_ffn,
    moe_forward,
    moe_forward_noalloc,
    moe_route,
    workspace_size,
)
