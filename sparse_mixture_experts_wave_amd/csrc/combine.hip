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

// K = top-k, a template parameter so that a thread loads every slot's row
// index and weight first and then has all 2K row loads in flight; the sums
// still run in slot order.  Indices are 32-bit: the entry points keep
// T * d below 2^31.
template <bool OUT_BF16, int K>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_sorted,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ topk_w,
                                                      const void* residual, void* y, int T, int d) {
  const int groups_per_row = d >> 3;
  const int total = T * groups_per_row;
  for (int g = blockIdx.x * blockDim.x + threadIdx.x; g < total; g += gridDim.x * blockDim.x) {
    const int t = g / groups_per_row;
    const int col = (g - t * groups_per_row) * 8;
    int row[K];
    float w[K];
#pragma unroll
    for (int s = 0; s < K; ++s) {
      row[s] = inv_pos[t * K + s];
      w[s] = topk_w[t * K + s];
    }
    float4 a[K], b[K];
#pragma unroll
    for (int s = 0; s < K; ++s) {
      if (row[s] >= 0) {
        const float4* src = reinterpret_cast<const float4*>(y_sorted + static_cast<int64_t>(row[s]) * d + col);
        a[s] = src[0];
        b[s] = src[1];
      }
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < K; ++s) {
      if (row[s] < 0) continue;
      acc[0] += w[s] * a[s].x; acc[1] += w[s] * a[s].y; acc[2] += w[s] * a[s].z; acc[3] += w[s] * a[s].w;
      acc[4] += w[s] * b[s].x; acc[5] += w[s] * b[s].y; acc[6] += w[s] * b[s].z; acc[7] += w[s] * b[s].w;
    }
    const int64_t off = static_cast<int64_t>(t) * d + col;
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
        const float4 ra = r[0], rb = r[1];
        acc[0] += ra.x; acc[1] += ra.y; acc[2] += ra.z; acc[3] += ra.w;
        acc[4] += rb.x; acc[5] += rb.y; acc[6] += rb.z; acc[7] += rb.w;
      }
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(y) + off);
      o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
}

template <bool OUT_BF16>
hipError_t launch_k(const float* y_sorted, const int32_t* inv_pos, const float* topk_w, const void* residual,
                    void* y, int T, int k, int d, unsigned blocks, hipStream_t s) {
#define MOE_COMBINE_K(KK)                                                                                  \
  case KK:                                                                                                \
    combine_kernel<OUT_BF16, KK><<<blocks, 256, 0, s>>>(y_sorted, inv_pos, topk_w, residual, y, T, d); \
    break;
  switch (k) {
    MOE_COMBINE_K(1)
    MOE_COMBINE_K(2)
    MOE_COMBINE_K(3)
    MOE_COMBINE_K(4)
    MOE_COMBINE_K(5)
    MOE_COMBINE_K(6)
    MOE_COMBINE_K(7)
    MOE_COMBINE_K(8)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_COMBINE_K
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float* y_sorted, const int32_t* inv_pos, const float* topk_w,
                          const void* residual, void* y, bool out_bf16, int64_t T, int k, int d,
                          hipStream_t stream) {
  if (T * d >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const int64_t groups = T * (d / 8);
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const unsigned nb = static_cast<unsigned>(blocks);
  const int Ti = static_cast<int>(T);
  return out_bf16 ? launch_k<true>(y_sorted, inv_pos, topk_w, residual, y, Ti, k, d, nb, stream)
                  : launch_k<false>(y_sorted, inv_pos, topk_w, residual, y, Ti, k, d, nb, stream);
}

}  // namespace moe
