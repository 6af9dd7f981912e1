// Host-side launchers of the gfx950 kernels.  Each returns the HIP status of
// its launch(es); none synchronises.  Shapes are validated by the C ABI layer
// (moe_api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace moe {

// Router GEMM + top-k (k <= kRouterMaxK) + softmax over the kept logits (optionally with a fused RMSNorm that
// also writes the normalised rows u in the activation dtype).
hipError_t launch_route(const void* x, bool x_bf16, const float* w_gate, const float* bias,
                        float* logits, int32_t* topk_idx, float* topk_w, int64_t T, int d,
                        int E, int k, const float* gamma, float eps, void* u_out, hipStream_t stream);
constexpr int kRouterMaxK = 8;

// Stable counting sort of (token, slot) pairs by expert.
hipError_t launch_dispatch(const int32_t* topk_idx, int64_t T, int k, int E,
                           int32_t* expert_offsets, int32_t* sorted_token, int32_t* inv_pos,
                           hipStream_t stream);

// Expert SwiGLU FFN over the dispatched rows, bf16 weights/activations, in two
// launches: up (h = SiLU(x W1^T + b1) * (x W3^T + b3), [T*k][d_ff] bf16) and
// down (y_sorted = h W2^T + b2, [T*k][d] fp32).  Each per-expert Linear bias
// ([E][d_ff] or [E][d], weight dtype) may be null.  Small T streams the weights.
// part: the GEMM path's partial-sum buffer (gemm_partial_bytes) or NULL, in
// which case the last round of tiles is not split.
hipError_t launch_expert_up_bf16(const uint16_t* x, const int32_t* expert_offsets,
                                 const int32_t* sorted_token, const uint16_t* w1,
                                 const uint16_t* w3, const uint16_t* b1, const uint16_t* b3,
                                 uint16_t* h, int64_t T, int k, int d, int d_ff, int E,
                                 float* part, hipStream_t stream);
hipError_t launch_expert_down_bf16(const uint16_t* h, const int32_t* expert_offsets,
                                   const uint16_t* w2, const uint16_t* b2, float* y_sorted, int64_t T,
                                   int k, int d, int d_ff, int E, float* part, hipStream_t stream);

// Same in fp32 (h is [T*k][d_ff] fp32).
hipError_t launch_expert_up_f32(const float* x, const int32_t* expert_offsets,
                                const int32_t* sorted_token, const float* w1, const float* w3,
                                const float* b1, const float* b3, float* h, int64_t T, int k, int d,
                                int d_ff, int E, hipStream_t stream);
hipError_t launch_expert_down_f32(const float* h, const int32_t* expert_offsets, const float* w2,
                                  const float* b2, float* y_sorted, int64_t T, int k, int d, int d_ff,
                                  int E, hipStream_t stream);

// Weighted gather-combine (+ optional residual), output in the activation dtype.
hipError_t launch_combine(const float* y_sorted, const int32_t* inv_pos, const float* topk_w,
                          const void* residual, void* y, bool out_bf16, int64_t T, int k, int d,
                          hipStream_t stream);

// Decode-regime streaming kernels (expert_stream.hip), used by the bf16
// launchers above when stream_supported(T, d, d_ff).
bool stream_supported(int64_t T, int d, int d_ff);
hipError_t launch_stream_up_bf16(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_token,
                                 const uint16_t* w1, const uint16_t* w3, const uint16_t* b1,
                                 const uint16_t* b3, uint16_t* h, int64_t T, int d, int d_ff, int E,
                                 hipStream_t stream);
hipError_t launch_stream_down_bf16(const uint16_t* h, const int32_t* offsets, const uint16_t* w2,
                                   const uint16_t* b2, float* y_sorted, int64_t T, int d, int d_ff,
                                   int E, hipStream_t stream);
// The streaming up projection with the dispatch folded in, for decode-size
// layers (stream_dispatch_supported: T * k <= 64 pairs, E <= 64): it sorts the
// router's topk_idx [T][k] itself and stores offsets, sorted_token and inv_pos
// as launch_dispatch would, so no dispatch launch precedes it.
bool stream_dispatch_supported(int64_t T, int k, int d, int d_ff, int E);
hipError_t launch_stream_up_dispatch_bf16(const uint16_t* x, const int32_t* topk_idx, int k, int32_t* offsets,
                                          int32_t* sorted_token, int32_t* inv_pos, const uint16_t* w1,
                                          const uint16_t* w3, const uint16_t* b1, const uint16_t* b3, uint16_t* h,
                                          int64_t T, int d, int d_ff, int E, hipStream_t stream);

// Prefill-regime grouped MFMA GEMMs (expert_gemm.hip).
hipError_t launch_gemm_up_bf16(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_token,
                               const uint16_t* w1, const uint16_t* w3, const uint16_t* b1,
                               const uint16_t* b3, uint16_t* h, int64_t T, int k, int d, int d_ff, int E,
                               float* part, hipStream_t stream);
hipError_t launch_gemm_down_bf16(const uint16_t* h, const int32_t* offsets, const uint16_t* w2,
                                 const uint16_t* b2, float* y_sorted, int64_t T, int k, int d, int d_ff,
                                 int E, float* part, hipStream_t stream);
// The down form with the residual connection fused into the epilogue: no fp32
// output; resid[rows][N] (bf16, row-contiguous) += a . w^T (+ b), one rounding.
hipError_t launch_gemm_down_residual_bf16(const uint16_t* a, const int32_t* offsets, const uint16_t* w,
                                          const uint16_t* b, uint16_t* resid, int64_t rows, int N, int K, int E,
                                          float* part, hipStream_t stream);
// The fused Q|K|V projection of attention (one expert owning all rows, no
// bias) with RoPE in the epilogue: q [rows][nq], k, v [rows][nkv] bf16 get the
// columns of a . w^T, q and k turned by cs [rows][64] (cos, sin) pairs of
// 128-wide heads.  nq and nkv are multiples of 128.
hipError_t launch_gemm_qkv_rope_bf16(const uint16_t* a, const int32_t* offsets, const uint16_t* w,
                                     const float* cs, uint16_t* q, uint16_t* k, uint16_t* v, int64_t rows, int nq,
                                     int nkv, int K, float* part, hipStream_t stream);

// Router load-balancing loss over [layers][T][E] logits (aux_loss.hip).
int aux_loss_max_k();
hipError_t launch_aux_loss(const float* logits, int64_t layers, int64_t T, int E, int k, const uint8_t* mask,
                           float alpha, float* loss, float* stats, hipStream_t stream);

// Attention sublayer (attention.hip): row RMSNorm (bf16 -> bf16; it also
// writes row_range = [0, T], the offsets that let the expert GEMM run one
// dense projection, and with cs set the RoPE table cs [T][64] (cos, sin) of
// positions pos0 + t for d_h = 128), RoPE + split of the fused Q|K|V
// projection (fp32 -> bf16 head-major), causal GQA flash attention (bf16,
// d_h = 128) and the residual add (h += y, one rounding).
hipError_t launch_rmsnorm_rows(const uint16_t* x, const float* gamma, float eps, uint16_t* u, int64_t T, int d,
                               int32_t* row_range, hipStream_t stream, float* cs = nullptr, double theta = 0.0,
                               int64_t pos0 = 0);
hipError_t launch_rope_pack(const float* qkv, uint16_t* q, uint16_t* k, uint16_t* v, int64_t T, int H, int G,
                            int dh, double theta, int64_t pos0, hipStream_t stream);
bool flash_attn_supported(int dh);
hipError_t launch_flash_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int64_t T,
                             int H, int G, int dh, hipStream_t stream);
hipError_t launch_residual_add(uint16_t* h, const float* y, int64_t n, hipStream_t stream);

// Token count at or below which the bf16 expert FFN streams weights
// (decode regime) instead of running the tiled grouped GEMM.
constexpr int64_t kStreamMaxT = 64;

// The grouped GEMM's partial-sum buffer: room for the K pieces of one round of
// split tiles, at most kGemmMaxPieces pieces of 256 x 256 fp32.
constexpr int kGemmMaxPieces = 256;
constexpr size_t kGemmPartialBytes = static_cast<size_t>(kGemmMaxPieces) * 256 * 256 * 4;
// Bytes of partial-sum buffer a bf16 expert FFN of this shape uses (0 when it
// takes the streaming path).
inline size_t gemm_partial_bytes(int64_t T, int d, int d_ff) {
  return stream_supported(T, d, d_ff) ? 0 : kGemmPartialBytes;
}

}  // namespace moe
