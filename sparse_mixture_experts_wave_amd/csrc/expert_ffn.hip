// Expert SwiGLU FFN over the dispatched rows:
//   h[r]        = SiLU(x[t] W1_e^T + b1_e) * (x[t] W3_e^T + b3_e)      t = sorted_token[r]
//   y_sorted[r] = h[r] W2_e^T + b2_e
// ("Mixtral" textbook page, "Прямой проход в формулах", MoE equation: the
// expert term (SiLU(u W_gate) * u W_up) W_down; w1 = gate, w3 = up, w2 = down
// per the page's HuggingFace weight mapping.  The Linear biases are optional:
// section "Конфигурация", key `bias`; Mixtral 8x7B has none.)
//
// Dispatch between the bf16 paths (decode-regime streaming kernel in
// expert_stream.hip, prefill-regime MFMA GEMM in expert_gemm.hip) and the
// fp32 path below: a plain LDS-tiled FMA GEMM for fp32 layers.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// fp32 grouped GEMM (plain FMA, LDS tiled)
// ---------------------------------------------------------------------------
constexpr int F_BM = 64;
constexpr int F_BN = 64;
constexpr int F_BK = 16;

template <bool GATED>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, int E, const float* __restrict__ B0,
    const float* __restrict__ B1, const float* __restrict__ bias0, const float* __restrict__ bias1,
    float* __restrict__ out, int N, int K) {
  __shared__ float As[F_BM][F_BK + 1];
  __shared__ float Bs0[F_BN][F_BK + 1];
  __shared__ float Bs1[GATED ? F_BN : 1][F_BK + 1];

  int first_row, rows;
  const int e = tile_to_expert<F_BM>(offsets, E, blockIdx.y, &first_row, &rows);
  if (e < 0) return;
  const int n0 = blockIdx.x * F_BN;
  const int tid = threadIdx.x;
  const int tx = tid & 15;
  const int ty = tid >> 4;

  const int lr = tid >> 2;        // row of the tile this thread copies
  const int lk = (tid & 3) * 4;   // first of its four k columns
  const bool a_ok = lr < rows;
  const int64_t a_row = a_ok ? (gather ? gather[first_row + lr] : first_row + lr) : 0;
  const bool b_ok = n0 + lr < N;
  const int64_t b_row = static_cast<int64_t>(e) * N + (b_ok ? n0 + lr : 0);

  float acc0[4][4] = {}, acc1[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += F_BK) {
    const float4 av = a_ok ? *reinterpret_cast<const float4*>(A + a_row * K + k0 + lk) : make_float4(0, 0, 0, 0);
    const float4 bv = b_ok ? *reinterpret_cast<const float4*>(B0 + b_row * K + k0 + lk) : make_float4(0, 0, 0, 0);
    As[lr][lk] = av.x; As[lr][lk + 1] = av.y; As[lr][lk + 2] = av.z; As[lr][lk + 3] = av.w;
    Bs0[lr][lk] = bv.x; Bs0[lr][lk + 1] = bv.y; Bs0[lr][lk + 2] = bv.z; Bs0[lr][lk + 3] = bv.w;
    if constexpr (GATED) {
      const float4 cv = b_ok ? *reinterpret_cast<const float4*>(B1 + b_row * K + k0 + lk) : make_float4(0, 0, 0, 0);
      Bs1[lr][lk] = cv.x; Bs1[lr][lk + 1] = cv.y; Bs1[lr][lk + 2] = cv.z; Bs1[lr][lk + 3] = cv.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < F_BK; ++kk) {
      float a[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[ty + 16 * i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = Bs0[tx + 16 * j][kk];
        if constexpr (GATED) b1[j] = Bs1[tx + 16 * j][kk];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0[i][j] += a[i] * b0[j];
          if constexpr (GATED) acc1[i][j] += a[i] * b1[j];
        }
    }
    __syncthreads();
  }
  float bb0[4], bb1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + tx + 16 * j;
    const int64_t bi = static_cast<int64_t>(e) * N + (n < N ? n : 0);
    bb0[j] = bias0 ? bias0[bi] : 0.f;
    bb1[j] = (GATED && bias1) ? bias1[bi] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = ty + 16 * i;
      const int n = n0 + tx + 16 * j;
      if (r < rows && n < N) {
        const int64_t o = static_cast<int64_t>(first_row + r) * N + n;
        out[o] = GATED ? silu_exact(acc0[i][j] + bb0[j]) * (acc1[i][j] + bb1[j]) : acc0[i][j] + bb0[j];
      }
    }
}

}  // namespace

hipError_t launch_expert_up_bf16(const uint16_t* x, const int32_t* expert_offsets,
                                 const int32_t* sorted_token, const uint16_t* w1,
                                 const uint16_t* w3, const uint16_t* b1, const uint16_t* b3,
                                 uint16_t* h, int64_t T, int k, int d, int d_ff, int E,
                                 float* part, hipStream_t stream) {
  if (stream_supported(T, d, d_ff))
    return launch_stream_up_bf16(x, expert_offsets, sorted_token, w1, w3, b1, b3, h, T, d, d_ff, E, stream);
  return launch_gemm_up_bf16(x, expert_offsets, sorted_token, w1, w3, b1, b3, h, T, k, d, d_ff, E, part, stream);
}

hipError_t launch_expert_down_bf16(const uint16_t* h, const int32_t* expert_offsets,
                                   const uint16_t* w2, const uint16_t* b2, float* y_sorted, int64_t T,
                                   int k, int d, int d_ff, int E, float* part, hipStream_t stream) {
  if (stream_supported(T, d, d_ff))
    return launch_stream_down_bf16(h, expert_offsets, w2, b2, y_sorted, T, d, d_ff, E, stream);
  return launch_gemm_down_bf16(h, expert_offsets, w2, b2, y_sorted, T, k, d, d_ff, E, part, stream);
}

hipError_t launch_expert_up_f32(const float* x, const int32_t* expert_offsets,
                                const int32_t* sorted_token, const float* w1, const float* w3,
                                const float* b1, const float* b3, float* h, int64_t T, int k, int d,
                                int d_ff, int E, hipStream_t stream) {
  const int64_t rows = T * k;
  const dim3 grid(static_cast<unsigned>((d_ff + F_BN - 1) / F_BN),
                  static_cast<unsigned>((rows + F_BM - 1) / F_BM + E));
  grouped_gemm_f32_kernel<true><<<grid, 256, 0, stream>>>(x, sorted_token, expert_offsets, E, w1, w3, b1, b3, h,
                                                          d_ff, d);
  return hipGetLastError();
}

hipError_t launch_expert_down_f32(const float* h, const int32_t* expert_offsets, const float* w2,
                                  const float* b2, float* y_sorted, int64_t T, int k, int d, int d_ff,
                                  int E, hipStream_t stream) {
  const int64_t rows = T * k;
  const dim3 grid(static_cast<unsigned>((d + F_BN - 1) / F_BN),
                  static_cast<unsigned>((rows + F_BM - 1) / F_BM + E));
  grouped_gemm_f32_kernel<false><<<grid, 256, 0, stream>>>(h, nullptr, expert_offsets, E, w2, nullptr, b2, nullptr,
                                                           y_sorted, d, d_ff);
  return hipGetLastError();
}

}  // namespace moe
