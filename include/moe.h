/*
 * moe.h - C ABI of the MI355X (gfx950) Mixtral sparse MoE feed-forward layer.
 *
 * The layer (the "Mixtral" textbook page, section "Научный вклад", layer
 * formula, and section "Прямой проход в формулах", MoE equation):
 *
 *     g   = x W_g                   router logits, one per expert
 *     S   = the k largest logits    (Mixtral: k = 2; the others count as -inf)
 *     w_i = e^{g_i} / sum_{j in S} e^{g_j}          (float32)
 *     y   = sum_{i in S} w_i (SiLU(x W1_i) * (x W3_i)) W2_i
 *
 * with W1 = gate, W3 = up, W2 = down (same page, section "Загрузка весов
 * HuggingFace").  The steps map onto the entry points as the page's
 * expert-major algorithm (section "Алгоритм") splits them: route, dispatch the
 * tokens of each expert, run each expert on its rows, combine the weighted
 * outputs back in token order.  Dropless: every token gets exactly k rows.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer is a device pointer, allocated and owned by the
 *   caller; the library allocates nothing and keeps no state between calls
 *   apart from cached device properties.  Inputs are read only; outputs are
 *   fully overwritten, never accumulated into.  Every non-NULL pointer must be
 *   16-byte aligned.
 * Layout.  Row-major, reduction dimension contiguous (nn.Linear):
 *   x [T][d], w_gate [E][d] fp32, w1 and w3 [E][d_ff][d], w2 [E][d][d_ff].
 *   bf16 values are raw 16-bit patterns (uint16).
 * Streams.  Every call is asynchronous on `stream` (a hipStream_t passed as
 *   void*; NULL is the default stream).  No call synchronises with the host
 *   or copies device data to the host, so sequences can be graph-captured.
 * Errors.  Arguments are validated on the host before anything is launched;
 *   a failed call launches nothing and sets a thread-local message readable
 *   with moe_last_error().  T == 0 returns MOE_OK without launching.
 *   MOE_ERR_INVALID_ARG: NULL/misaligned pointer, T < 0, d or d_ff not a
 *     positive multiple of 64 (d <= 32768, d_ff <= 65536), E outside 2..64,
 *     k outside 1..E (the pages' constructor raises ValueError for this),
 *     workspace too small.
 *   MOE_ERR_UNSUPPORTED: k > 8, E not a power of two, T * d >= 2^31, or an
 *     (act, wt) dtype pair other than (F32, F32) and (BF16, BF16).
 *   MOE_ERR_HIP: a HIP launch failed.
 * Precision.  Router logits, the top-k softmax and the combine weights are
 *   fp32 (the pages compute the router softmax in float32).  Expert GEMMs
 *   accumulate in fp32; with bf16 weights the SwiGLU intermediate h is
 *   rounded to bf16 and y_sorted is fp32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_HIP = 3
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer shape.  The pages' constructor arguments: T = batch * seq tokens,
 * d = emb_size, d_ff = hidden_dim, E = num_experts, k = top_k_experts.
 * act is the dtype of x / y (and of the residual stream), wt of w1/w3/w2. */
typedef struct {
  int64_t T;
  int32_t d;
  int32_t d_ff;
  int32_t E;
  int32_t k;
  int32_t act; /* moe_dtype */
  int32_t wt;  /* moe_dtype */
} moe_shape;

/* Optional per-expert Linear biases ("Mixtral" page, section "Конфигурация":
 * the `bias` key puts a bias on every Linear, the experts' included; it is on
 * by default there and off in Mixtral 8x7B).  With them an expert computes
 *   (SiLU(u W1_e^T + b1_e) * (u W3_e^T + b3_e)) W2_e^T + b2_e.
 * Each pointer may be NULL (that projection has no bias), and so may the
 * struct itself.  Device memory in the weight dtype wt, 16-byte aligned,
 * owned by the caller, read only:
 *   b1, b3  [E][d_ff]   (gate, up)
 *   b2      [E][d]      (down)                                              */
typedef struct {
  const void* b1;
  const void* b3;
  const void* b2;
} moe_expert_bias;

/* Bytes of workspace moe_forward and moe_block_forward need (256-byte
 * aligned sub-buffers: routing, permutation, h [T*k][d_ff] in wt, y_sorted
 * [T*k][d] fp32, for the block form the normalised input, and when the bf16
 * grouped GEMM runs (T > 64) a fixed 64 MiB of fp32 partial sums: the last
 * round of GEMM tiles is split along K over the idle CUs and summed in a
 * fixed order, so results stay deterministic).  Returns 0 for an invalid
 * shape.  Host only. */
size_t moe_workspace_size(const moe_shape* shape);

/* Bytes of workspace moe_expert_ffn needs (h, then the GEMM partial sums as
 * above).  Host only. */
size_t moe_expert_ffn_workspace_size(const moe_shape* shape);

/* Router: logits g = x W_g^T (+ bias), the k largest per token (k <= 8) and
 * their softmax weights.  ("Mixtral" page, "Прямой проход в формулах", MoE
 * equation; "MoE изнутри" steps 1-2.)
 *   x        [T][d] in act
 *   w_gate   [E][d] fp32
 *   bias     [E] fp32 or NULL (Mixtral has none; a Linear bias otherwise)
 *   logits   [T][E] fp32 output or NULL
 *   topk_idx [T][k] int32 output: slots in descending logit order; exactly
 *            equal logits go to the lower expert index
 *   topk_w   [T][k] fp32 output, sums to 1 per token                    */
moe_status moe_route(const moe_shape* shape, const void* x, const float* w_gate,
                     const float* bias, float* logits, int32_t* topk_idx,
                     float* topk_w, void* stream);

/* Dispatch: stable counting sort of the T*k (token, slot) pairs by expert,
 * the order in which the pages' expert loop visits them ("Алгоритм"):
 * expert by expert, each expert's tokens ascending.
 *   topk_idx       [T][k] int32, entries in 0..E-1 (others are skipped and
 *                  get inv_pos -1)
 *   expert_offsets [E+1] int32 output: rows of expert e are
 *                  [offsets[e], offsets[e+1]); empty experts get no rows
 *   sorted_token   [T*k] int32 output: token of each row, ascending per expert
 *   inv_pos        [T][k] int32 output: row holding (t, topk_idx[t][s])
 *   ws, ws_bytes   unused, may be NULL / 0                                 */
moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_idx,
                        int32_t* expert_offsets, int32_t* sorted_token,
                        int32_t* inv_pos, void* ws, size_t ws_bytes, void* stream);

/* Experts: for every row r of expert e (in dispatch order),
 *   y_sorted[r] = (SiLU(x[t] W1_e^T) * (x[t] W3_e^T)) W2_e^T,  t = sorted_token[r]
 * ("Прямой проход в формулах", MoE equation, the SwiGLU term), plus the
 * expert's Linear biases when expert_bias gives them (see moe_expert_bias).
 *   x             [T][d] in act;  w1, w3 [E][d_ff][d], w2 [E][d][d_ff] in wt
 *   expert_bias   NULL or biases (see above)
 *   y_sorted      [T*k][d] fp32 output
 *   ws            >= moe_expert_ffn_workspace_size(shape) bytes
 * Small T (<= 64, bf16) runs the weight-streaming path that reads each
 * touched expert's weights once; larger T runs the grouped MFMA GEMM.       */
moe_status moe_expert_ffn(const moe_shape* shape, const void* x,
                          const int32_t* expert_offsets, const int32_t* sorted_token,
                          const void* w1, const void* w3, const void* w2,
                          const moe_expert_bias* expert_bias, float* y_sorted,
                          void* ws, size_t ws_bytes, void* stream);

/* Combine: y[t] = sum_s topk_w[t][s] * y_sorted[inv_pos[t][s]] (+ residual[t]),
 * in fp32, rounded once to act ("Алгоритм", the weighted index-add, done as
 * a gather so no atomics are needed).
 *   residual [T][d] in act or NULL; may alias y.  Rows with inv_pos < 0 are
 *   skipped.                                                               */
moe_status moe_combine(const moe_shape* shape, const float* y_sorted,
                       const int32_t* inv_pos, const float* topk_w,
                       const void* residual, void* y, void* stream);

/* The whole layer: route -> dispatch -> experts -> combine on one stream.
 *   bias         router bias [E] fp32 or NULL (as in moe_route)
 *   expert_bias  NULL or the experts' Linear biases (moe_expert_bias)
 *   y [T][d] in act output (must not alias x)
 *   ws >= moe_workspace_size(shape) bytes                                   */
moe_status moe_forward(const moe_shape* shape, const void* x, const float* w_gate,
                       const float* bias, const void* w1, const void* w3,
                       const void* w2, const moe_expert_bias* expert_bias,
                       void* y, void* ws, size_t ws_bytes, void* stream);

/* The whole layer exactly as moe_forward, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument.  The routing,
 * the permutation, h [T*k][d_ff] and y_sorted [T*k][d] live instead in a
 * static 64 MiB device buffer inside the library, one per GPU, held until
 * the process ends.  The call allocates nothing.
 *   Arguments and errors as moe_forward (y must not alias x).
 *   Limit: those intermediates must fit 64 MiB.  At Mixtral's shape (d 4096,
 *   d_ff 14336, bf16, k 2) that is T <= 744 tokens; a larger T returns
 *   MOE_ERR_UNSUPPORTED and launches nothing.
 *   Sharing: every call on a GPU uses that GPU's one buffer and leaves its
 *   contents there; calls that overlap on one GPU (other streams, other
 *   threads) race and must be serialised by the caller.  Nothing in the
 *   buffer needs to start zeroed.
 *   Results: bit-identical to moe_forward on the streaming path (bf16,
 *   T <= 64) and the fp32 path; on the bf16 GEMM path the last round of GEMM
 *   tiles is not split along K (moe_forward keeps those partial sums in its
 *   workspace), so the fp32 sums run in another order.                      */
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_gate,
                               const float* bias, const void* w1, const void* w3,
                               const void* w2, const moe_expert_bias* expert_bias,
                               void* y, void* stream);

/* One pre-norm residual MoE sublayer ("Прямой проход в формулах", block
 * equation H = U + MoE(RMSNorm_2(U)); RMSNorm(z) = z / sqrt(mean z^2 + eps)
 * * gamma), in place on h:
 *   h_inout [T][d] in act, overwritten with h + MoE(RMSNorm(h))
 *   gamma   [d] fp32;  eps > 0
 * The router's logits are rinv * sum_j (h_j gamma_j) W[e][j] with rinv the fp32
 * inverse root of the fp32 mean square (the normalised row before rounding);
 * the experts see the normalised row rounded to act. */
moe_status moe_block_forward(const moe_shape* shape, void* h_inout, const float* gamma,
                             float eps, const float* w_gate, const float* bias,
                             const void* w1, const void* w3, const void* w2,
                             const moe_expert_bias* expert_bias,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * The attention sublayer around the MoE ("Mixtral" page, section "Прямой
 * проход в формулах": U = H + GQA(RMSNorm_1(H)) with
 *   Q_h = RoPE(X W_Q^h), K_c = RoPE(X W_K^c), V_c = X W_V^c,
 *   O_h = softmax(Q_h K_kappa(h)^T / sqrt(d_h) + M) V_kappa(h),
 *   kappa(h) = h / (H / G), M the causal mask,
 *   GQA(X) = [O_0; ...; O_{H-1}] W_O).
 * RoPE turns the pair (2i, 2i+1) of a head vector at position p by the angle
 * p * rope_theta^(-2i / d_h) (the interleaved form the page's HF loader
 * implies by permuting q_proj / k_proj rows).  One sequence of T new tokens
 * at positions pos0 .. pos0 + T - 1, no KV cache, no sliding window.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t T;    /* tokens of the sequence */
  int32_t d;    /* model width, a positive multiple of 64 */
  int32_t H;    /* query heads */
  int32_t G;    /* key / value groups, H % G == 0 */
  int32_t d_h;  /* head dimension: 128 is implemented */
  int32_t act;  /* moe_dtype of activations and weights: BF16 is implemented */
} moe_attn_shape;

/* Bytes of workspace moe_attention_block_forward needs: the normalised
 * input, the rotated heads and the attention output; for T > 64 the GEMM
 * partial sums as for moe_workspace_size and a [T][64] table of RoPE
 * (cos, sin) pairs (the projections' epilogues rotate and add into h
 * directly); for T <= 64 the fp32 Q|K|V and output projections instead.
 * 0 for an invalid or unsupported shape.  Host only. */
size_t moe_attention_workspace_size(const moe_attn_shape* shape);

/* Causal GQA attention core on rotated heads:
 *   O_h[t] = sum_{s <= t} softmax_s(Q_h[t] . K_kappa(h)[s] / sqrt(d_h)) V_kappa(h)[s]
 *   q [T][H][d_h], k, v [T][G][d_h], o [T][H][d_h] output, all act (bf16).
 * Errors as for the MoE calls: MOE_ERR_INVALID_ARG for H % G != 0, odd or
 * non-positive d_h, NULL / misaligned pointers; MOE_ERR_UNSUPPORTED for
 * d_h != 128, act != BF16 or T * (H + 2G) * d_h >= 2^31.                     */
moe_status moe_gqa_attention(const moe_attn_shape* shape, const void* q, const void* k,
                             const void* v, void* o, void* stream);

/* The whole sublayer, in place: h <- h + GQA(RMSNorm(h) * gamma).
 *   h_inout  [T][d] act
 *   gamma    [d] fp32;  eps > 0
 *   wqkv     [(H + 2G) d_h][d] act: the rows of W_Q ([H d_h][d]), then W_K,
 *            then W_V ([G d_h][d] each), nn.Linear layout (the pages' three
 *            Linear weights stacked row-wise)
 *   wo       [d][H d_h] act
 *   rope_theta > 0 (Mixtral 8x7B: 1e6);  pos0 >= 0
 *   ws >= moe_attention_workspace_size(shape) bytes                          */
moe_status moe_attention_block_forward(const moe_attn_shape* shape, void* h_inout,
                                       const float* gamma, float eps, const void* wqkv,
                                       const void* wo, float rope_theta, int64_t pos0,
                                       void* ws, size_t ws_bytes, void* stream);

/* Router load-balancing loss ("Mixtral" page, section "Load-balancing
 * loss"): L_aux = alpha * E * sum_{s<k} sum_i f_{s,i} * P_i, where f_{s,i} is
 * the share of tokens whose s-th largest logit is expert i (ties -> lower
 * index) and P_i the mean over tokens of the softmax over all E logits; the
 * statistics pool all layers and every token with a nonzero mask byte.
 *   logits     [num_layers][T][E] fp32 (the router logits of each layer,
 *              e.g. from moe_route's logits output)
 *   token_mask [T] uint8 or NULL (all tokens); the same mask for every layer
 *   loss       [1] fp32 output;  stats [(k+1)*E] fp32 output or NULL:
 *              f_{s,i} at s*E + i, then P_i at k*E + i
 * Uses shape->T, E, k (1 <= k <= min(E, 8); any d, d_ff, dtypes).  One
 * workgroup; the result is bitwise deterministic.  Zero valid tokens give 0. */
moe_status moe_aux_loss(const moe_shape* shape, const float* logits, int32_t num_layers,
                        const uint8_t* token_mask, float alpha, float* loss, float* stats,
                        void* stream);

/* Timing points.  After a successful call with MOE_TIMING_POINTS events,
 * every moe_forward / moe_block_forward on the calling thread records
 * events[i] on its stream at point i:
 *   0 before the router   1 after the router   2 after dispatch
 *   3 after the expert up kernel (h)   4 after the expert down kernel
 *   5 after the combine
 * so the elapsed time between consecutive points is one kernel's duration
 * on that stream.  events are hipEvent_t handles created and owned by the
 * caller; they must outlive their use.  count 0 or events NULL stops the
 * recording.  Host only; thread-local.  MOE_ERR_INVALID_ARG for another
 * count or a NULL handle. */
#define MOE_TIMING_POINTS 6
moe_status moe_set_timing_events(void* const* events, int32_t count);

/* Message of the last non-OK status on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
