// Expert SwiGLU FFN over the dispatched rows:
//   h[r]        = SiLU(x[t] W1_e^T) * (x[t] W3_e^T)      t = sorted_token[r]
//   y_sorted[r] = h[r] W2_e^T
// ("Mixtral" textbook page, "Прямой проход в формулах", MoE equation: the
// expert term (SiLU(u W_gate) * u W_up) W_down; w1 = gate, w3 = up, w2 = down
// per the page's HuggingFace weight mapping.)
//
// Three code paths:
//  * grouped_gemm_bf16: tiled bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16),
//    128x128 output tiles per 256-thread workgroup, K staged through LDS in
//    64-wide double-buffered slices with an XOR swizzle on 16-byte chunks.
//    The up kernel computes the gate and up tiles of the same columns in one
//    pass and applies SiLU(gate) * up in the epilogue, so only h is written.
//    M-tiles are numbered across experts (ceil(n_e / 128) per expert); each
//    workgroup finds its expert from the offsets, so no tile map is stored.
//  * stream_ffn_bf16: decode regime (few rows per expert).  Every touched
//    expert's weights are read exactly once, straight from HBM into MFMA
//    operands (v_mfma_f32_16x16x32_bf16, 16 rows of the expert per block);
//    the four waves of a workgroup split K and reduce through LDS.
//  * grouped_gemm_f32: plain LDS-tiled fp32 FMA GEMM for fp32 layers.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// bf16 grouped GEMM (prefill regime)
// ---------------------------------------------------------------------------
constexpr int GM_BM = 128;
constexpr int GM_BN = 128;
constexpr int GM_BK = 64;

// Element offset of 16-byte chunk c of row r inside a [rows][64] bf16 LDS tile.
__device__ __forceinline__ int swz(int r, int c) { return r * GM_BK + ((c ^ (r & 7)) << 3); }

template <bool GATED>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, void* __restrict__ out, int N, int K) {
  constexpr int NMAT = GATED ? 3 : 2;
  constexpr int TILE = GM_BM * GM_BK;  // elements per operand tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][NMAT * TILE];

  int first_row, rows;
  const int e = tile_to_expert<GM_BM>(offsets, E, blockIdx.y, &first_row, &rows);
  if (e < 0) return;
  const int n0 = blockIdx.x * GM_BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = tid & 7;

  // Global->LDS assignment: thread copies chunk `chunk` of rows tid/8 + 32 i.
  const uint16_t* a_src[4];
  const uint16_t* b0_src[4];
  const uint16_t* b1_src[4];
  bool a_ok[4], b_ok[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    a_ok[i] = r < rows;
    int src = 0;
    if (a_ok[i]) src = gather ? gather[first_row + r] : first_row + r;
    a_src[i] = A + static_cast<int64_t>(src) * K + chunk * 8;
    const int n = n0 + r;
    b_ok[i] = n < N;
    const int64_t brow = static_cast<int64_t>(e) * N + (b_ok[i] ? n : 0);
    b0_src[i] = B0 + brow * K + chunk * 8;
    b1_src[i] = GATED ? B1 + brow * K + chunk * 8 : nullptr;
    lds_off[i] = swz(r, chunk);
  }

  u32x4 ra[4], rb0[4], rb1[4];
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto gload = [&](int kt) {
    const int k0 = kt * GM_BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = a_ok[i] ? load16(a_src[i] + k0) : zero;
      rb0[i] = b_ok[i] ? load16(b0_src[i] + k0) : zero;
      if constexpr (GATED) rb1[i] = b_ok[i] ? load16(b1_src[i] + k0) : zero;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      store16(&smem[buf][lds_off[i]], ra[i]);
      store16(&smem[buf][TILE + lds_off[i]], rb0[i]);
      if constexpr (GATED) store16(&smem[buf][2 * TILE + lds_off[i]], rb1[i]);
    }
  };

  f32x16 acc0[2][2], acc1[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc0[mi][ni][v] = 0.f;
        acc1[mi][ni][v] = 0.f;
      }
    }

  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int KT = K / GM_BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint16_t* As = smem[cur];
    const uint16_t* Bs0 = smem[cur] + TILE;
    const uint16_t* Bs1 = smem[cur] + 2 * TILE;
#pragma unroll
    for (int kk = 0; kk < GM_BK / 16; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      bf16x8 a[2], b0[2], b1[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int r = wm * 64 + mi * 32 + (lane & 31);
        a[mi] = as_bf16x8(load16(As + swz(r, c)));
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int r = wn * 64 + ni * 32 + (lane & 31);
        b0[ni] = as_bf16x8(load16(Bs0 + swz(r, c)));
        if constexpr (GATED) b1[ni] = as_bf16x8(load16(Bs1 + swz(r, c)));
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          acc0[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b0[ni], acc0[mi][ni], 0, 0, 0);
          if constexpr (GATED)
            acc1[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b1[ni], acc1[mi][ni], 0, 0, 0);
        }
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column lane%32 and rows
  // 8*(v/4) + 4*(lane/32) + v%4 for v = 0..15.
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int n = n0 + wn * 64 + ni * 32 + (lane & 31);
        if (r < rows && n < N) {
          const int64_t o = static_cast<int64_t>(first_row + r) * N + n;
          if constexpr (GATED) {
            static_cast<uint16_t*>(out)[o] = f32_to_bf16(silu_fast(acc0[mi][ni][v]) * acc1[mi][ni][v]);
          } else {
            static_cast<float*>(out)[o] = acc0[mi][ni][v];
          }
        }
      }
}

// ---------------------------------------------------------------------------
// bf16 weight-streaming FFN (decode regime)
// ---------------------------------------------------------------------------
// Workgroup = expert blockIdx.y x 32 output columns (two 16-column groups).
// Wave w covers K range [w K/4, (w+1) K/4) in 128-wide steps: lane
// (m = lane%16, q = lane/16) loads bytes of k-chunk q of each 32-wide MFMA
// step, i.e. 64 contiguous bytes per weight row per load instruction.
template <int MB, bool GATED>
__global__ __launch_bounds__(256) void stream_ffn_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, void* __restrict__ out, int N, int K) {
  constexpr int NG = 2;
  constexpr int NACC = MB * NG * (GATED ? 2 : 1);
  __shared__ f32x4 red[3][NACC][64];

  const int e = blockIdx.y;
  const int lo = offsets[e];
  const int n_e = offsets[e + 1] - lo;
  if (n_e <= 0) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15;
  const int q = lane >> 4;
  const int n0 = blockIdx.x * (16 * NG);
  const int Kw = K >> 2;
  const int kb = wave * Kw;

  const uint16_t* b0row[NG];
  const uint16_t* b1row[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int64_t n = static_cast<int64_t>(e) * N + n0 + 16 * g + m;
    b0row[g] = B0 + n * K + kb + 8 * q;
    b1row[g] = GATED ? B1 + n * K + kb + 8 * q : nullptr;
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};

  for (int rb = 0; rb < n_e; rb += 16 * MB) {
    const uint16_t* arow[MB];
    bool aok[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = rb + mb * 16 + m;
      aok[mb] = r < n_e;
      int src = 0;
      if (aok[mb]) src = gather ? gather[lo + r] : lo + r;
      arow[mb] = A + static_cast<int64_t>(src) * K + kb + 8 * q;
    }
    f32x4 acc0[MB][NG], acc1[MB][NG];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc0[mb][g][v] = 0.f;
          acc1[mb][g][v] = 0.f;
        }

    for (int k = 0; k < Kw; k += 128) {
      u32x4 w0[NG][4], w1[NG][4], xa[MB][4];
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w0[g][j] = load16(b0row[g] + k + 32 * j);
          if constexpr (GATED) w1[g][j] = load16(b1row[g] + k + 32 * j);
        }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[mb][j] = aok[mb] ? load16(arow[mb] + k + 32 * j) : zero;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            acc0[mb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[mb][j]), as_bf16x8(w0[g][j]),
                                                                  acc0[mb][g], 0, 0, 0);
            if constexpr (GATED)
              acc1[mb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[mb][j]), as_bf16x8(w1[g][j]),
                                                                    acc1[mb][g], 0, 0, 0);
          }
    }

    // Reduce the four K quarters through LDS into wave 0.
    if (wave > 0) {
      int a = 0;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          red[wave - 1][a++][lane] = acc0[mb][g];
          if constexpr (GATED) red[wave - 1][a++][lane] = acc1[mb][g];
        }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        int a = 0;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            acc0[mb][g] += red[w][a++][lane];
            if constexpr (GATED) acc1[mb][g] += red[w][a++][lane];
          }
      }
      // 16x16 accumulator layout: lane holds column lane%16, rows 4*(lane/16)+v.
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = rb + mb * 16 + 4 * q + v;
            if (r < n_e) {
              const int64_t o = static_cast<int64_t>(lo + r) * N + n0 + 16 * g + m;
              if constexpr (GATED)
                static_cast<uint16_t*>(out)[o] = f32_to_bf16(silu_fast(acc0[mb][g][v]) * acc1[mb][g][v]);
              else
                static_cast<float*>(out)[o] = acc0[mb][g][v];
            }
          }
    }
    __syncthreads();
  }
}

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
    const float* __restrict__ B1, float* __restrict__ out, int N, int K) {
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
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = ty + 16 * i;
      const int n = n0 + tx + 16 * j;
      if (r < rows && n < N) {
        const int64_t o = static_cast<int64_t>(first_row + r) * N + n;
        out[o] = GATED ? silu_exact(acc0[i][j]) * acc1[i][j] : acc0[i][j];
      }
    }
}

}  // namespace

namespace {
bool use_stream(int64_t T, int d, int d_ff) {
  // n_e <= T for every expert (the top-k experts of a token are distinct).
  return T <= kStreamMaxT && d % 512 == 0 && d_ff % 512 == 0;
}
}  // namespace

hipError_t launch_expert_up_bf16(const uint16_t* x, const int32_t* expert_offsets,
                                 const int32_t* sorted_token, const uint16_t* w1,
                                 const uint16_t* w3, uint16_t* h, int64_t T, int k, int d,
                                 int d_ff, int E, hipStream_t stream) {
  if (use_stream(T, d, d_ff)) {
    const dim3 grid(static_cast<unsigned>(d_ff / 32), static_cast<unsigned>(E));
    if (T <= 16)
      stream_ffn_bf16_kernel<1, true><<<grid, 256, 0, stream>>>(x, sorted_token, expert_offsets, w1, w3, h, d_ff, d);
    else if (T <= 32)
      stream_ffn_bf16_kernel<2, true><<<grid, 256, 0, stream>>>(x, sorted_token, expert_offsets, w1, w3, h, d_ff, d);
    else
      stream_ffn_bf16_kernel<4, true><<<grid, 256, 0, stream>>>(x, sorted_token, expert_offsets, w1, w3, h, d_ff, d);
    return hipGetLastError();
  }
  const int64_t rows = T * k;
  const dim3 grid(static_cast<unsigned>((d_ff + GM_BN - 1) / GM_BN),
                  static_cast<unsigned>((rows + GM_BM - 1) / GM_BM + E));
  grouped_gemm_bf16_kernel<true><<<grid, 256, 0, stream>>>(x, sorted_token, expert_offsets, E, w1, w3, h, d_ff, d);
  return hipGetLastError();
}

hipError_t launch_expert_down_bf16(const uint16_t* h, const int32_t* expert_offsets,
                                   const uint16_t* w2, float* y_sorted, int64_t T, int k, int d,
                                   int d_ff, int E, hipStream_t stream) {
  if (use_stream(T, d, d_ff)) {
    const dim3 grid(static_cast<unsigned>(d / 32), static_cast<unsigned>(E));
    if (T <= 16)
      stream_ffn_bf16_kernel<1, false><<<grid, 256, 0, stream>>>(h, nullptr, expert_offsets, w2, nullptr, y_sorted, d, d_ff);
    else if (T <= 32)
      stream_ffn_bf16_kernel<2, false><<<grid, 256, 0, stream>>>(h, nullptr, expert_offsets, w2, nullptr, y_sorted, d, d_ff);
    else
      stream_ffn_bf16_kernel<4, false><<<grid, 256, 0, stream>>>(h, nullptr, expert_offsets, w2, nullptr, y_sorted, d, d_ff);
    return hipGetLastError();
  }
  const int64_t rows = T * k;
  const dim3 grid(static_cast<unsigned>((d + GM_BN - 1) / GM_BN),
                  static_cast<unsigned>((rows + GM_BM - 1) / GM_BM + E));
  grouped_gemm_bf16_kernel<false><<<grid, 256, 0, stream>>>(h, nullptr, expert_offsets, E, w2, nullptr, y_sorted, d, d_ff);
  return hipGetLastError();
}

hipError_t launch_expert_up_f32(const float* x, const int32_t* expert_offsets,
                                const int32_t* sorted_token, const float* w1, const float* w3,
                                float* h, int64_t T, int k, int d, int d_ff, int E,
                                hipStream_t stream) {
  const int64_t rows = T * k;
  const dim3 grid(static_cast<unsigned>((d_ff + F_BN - 1) / F_BN),
                  static_cast<unsigned>((rows + F_BM - 1) / F_BM + E));
  grouped_gemm_f32_kernel<true><<<grid, 256, 0, stream>>>(x, sorted_token, expert_offsets, E, w1, w3, h, d_ff, d);
  return hipGetLastError();
}

hipError_t launch_expert_down_f32(const float* h, const int32_t* expert_offsets, const float* w2,
                                  float* y_sorted, int64_t T, int k, int d, int d_ff, int E,
                                  hipStream_t stream) {
  const int64_t rows = T * k;
  const dim3 grid(static_cast<unsigned>((d + F_BN - 1) / F_BN),
                  static_cast<unsigned>((rows + F_BM - 1) / F_BM + E));
  grouped_gemm_f32_kernel<false><<<grid, 256, 0, stream>>>(h, nullptr, expert_offsets, E, w2, nullptr, y_sorted, d, d_ff);
  return hipGetLastError();
}

}  // namespace moe
