// Weighted gather-combine: y[t] = sum_s w[t][s] * y_sorted[inv_pos[t][s]]
// (+ residual[t]), fp32 arithmetic, one rounding to the activation dtype.
//
// This is the combine of the expert-major algorithm on the "Mixtral"
// textbook page (section "Алгоритм": index-add of the weighted expert
// outputs into Y), done as a gather so each output element is written once,
// without atomics, in slot order.  HBM-bound: each thread moves 8 columns
// (two 16-byte loads per source row, one 16-byte bf16 or two fp32 stores).
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_sorted,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ topk_w,
                                                      const void* residual, void* y, int64_t T,
                                                      int k, int d) {
  const int groups_per_row = d >> 3;
  const int64_t total = T * groups_per_row;
  for (int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; g < total;
       g += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = g / groups_per_row;
    const int col = static_cast<int>(g - t * groups_per_row) * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int s = 0; s < k; ++s) {
      const int row = inv_pos[t * k + s];
      if (row < 0) continue;
      const float w = topk_w[t * k + s];
      const float4* src = reinterpret_cast<const float4*>(y_sorted + static_cast<int64_t>(row) * d + col);
      const float4 a = src[0], b = src[1];
      acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
      acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
    }
    const int64_t off = t * d + col;
    if constexpr (OUT_BF16) {
      if (residual != nullptr) {
        const u32x4 r = load16(static_cast<const uint16_t*>(residual) + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += lo_bf16(r[i]);
          acc[2 * i + 1] += hi_bf16(r[i]);
        }
      }
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
      store16(static_cast<uint16_t*>(y) + off, o);
    } else {
      if (residual != nullptr) {
        const float4* r = reinterpret_cast<const float4*>(static_cast<const float*>(residual) + off);
        const float4 a = r[0], b = r[1];
        acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
        acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
      }
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(y) + off);
      o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y_sorted, const int32_t* inv_pos, const float* topk_w,
                          const void* residual, void* y, bool out_bf16, int64_t T, int k, int d,
                          hipStream_t stream) {
  const int64_t groups = T * (d / 8);
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (out_bf16)
    combine_kernel<true><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(y_sorted, inv_pos, topk_w, residual, y, T, k, d);
  else
    combine_kernel<false><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(y_sorted, inv_pos, topk_w, residual, y, T, k, d);
  return hipGetLastError();
}

}  // namespace moe
