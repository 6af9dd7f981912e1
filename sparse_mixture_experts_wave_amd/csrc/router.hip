// Router: g = x W_g^T (+ bias) in fp32, the k largest logits per token
// (k <= 8; Mixtral uses 2) and the softmax over them.  ("Mixtral" textbook page, "Прямой проход в
// формулах", MoE equation; "MoE изнутри", steps 1-2: Linear router, top-k,
// softmax over the kept logits in float32.)
//
// A workgroup handles TPB tokens; its NW waves split the row into NW equal
// parts (NW = 8 for one token per workgroup and E <= 16, so each wave's
// loads go out in a single pass; otherwise 4).  Each lane walks its part in
// 8-element (16-byte bf16) chunks, so a wave reads 1 KiB of a row per step,
// and every router weight chunk it
// loads serves all TPB tokens.  The TPB x E partial dot products are
// transposed through LDS: lane j of each wave sums column j over its 64
// lanes, then wave 0 adds the NW parts in order, so lane j ends with the logit
// of (token j / E, expert j % E).  The top-k is a butterfly over the E lanes
// of each token (E is a power of two), one round per kept expert.  Small T
// uses one token per workgroup
// so that T workgroups share the work.
//
// Precision: every product x_j * W[e][j] (bf16 or fp32 times fp32) is exact
// in fp64, and the sums are kept in fp64 until the logit is rounded once to
// fp32 (the pages fix the router's precision, fp32, not an order).  The fp64
// sum of d products is not exact itself: its relative error is at most about
// d * 2^-53, far below fp32's 2^-24, so the logit is the correctly rounded
// fp32 value of the exact dot product except when that value lies within
// the fp64 error of a rounding boundary between two fp32 numbers; then the
// summation order can move it by one fp32 ulp.  Such a 1-ulp difference can
// only change the top-k choice of a token whose logits are that close.
//
// With gamma != nullptr the kernel also applies RMSNorm: it accumulates
// sum(x^2) next to the dot products, and since u = x * rinv * gamma the
// logits are rinv * sum_j (x_j gamma_j) W[e][j], with rinv the fp32 inverse
// root of the fp32-rounded mean square: the product with rinv is formed in
// fp64 and rounded once.  The normalised rows u are then written (rounded to
// the activation dtype) for the experts.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

template <bool XBF16>
__device__ __forceinline__ void load_x8(const void* x, int64_t off, float v[8]) {
  if constexpr (XBF16) {
    const u32x4 w = load16(static_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = lo_bf16(w[i]);
      v[2 * i + 1] = hi_bf16(w[i]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

constexpr int MAX_K = 8;  // largest top-k the router supports

// (v, i) beats (w, j) when larger, or equal with the lower index.
__device__ __forceinline__ bool beats(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

template <int E, int TPB, int NW, bool XBF16, bool NORM>
__global__ __launch_bounds__(64 * NW) void router_top2_kernel(
    const void* __restrict__ x, const float* __restrict__ wg, const float* __restrict__ bias,
    const float* __restrict__ gamma, float eps, void* __restrict__ u_out,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int T, int d, int k) {
  constexpr int P = TPB * E;                   // logits per workgroup (<= 64)
  constexpr int COLS = P + (NORM ? TPB : 0);   // + sum of squares per token
  constexpr int LD = COLS + 1;                 // padded LDS row
  __shared__ double red[NW][64 * LD];
  __shared__ double part[NW][COLS];
  __shared__ float rinv_s[TPB];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tok0 = blockIdx.x * TPB;
  const int part_len = d / NW;  // a multiple of 8 (d % 64 == 0)
  const int cbeg = wave * part_len;
  const int cend = cbeg + part_len;

  double acc[TPB][E];
  double ss[TPB];
#pragma unroll
  for (int t = 0; t < TPB; ++t) {
    ss[t] = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[t][e] = 0.0;
  }

  for (int base = cbeg; base < cend; base += 512) {
    const int col = base + lane * 8;
    if (col < cend) {
      float xv[TPB][8];
#pragma unroll
      for (int t = 0; t < TPB; ++t) {
        if (tok0 + t < T) {
          load_x8<XBF16>(x, static_cast<int64_t>(tok0 + t) * d + col, xv[t]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[t][i] = 0.f;
        }
      }
      if constexpr (NORM) {
        const float4 g0 = *reinterpret_cast<const float4*>(gamma + col);
        const float4 g1 = *reinterpret_cast<const float4*>(gamma + col + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
        for (int t = 0; t < TPB; ++t)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            ss[t] += static_cast<double>(xv[t][i]) * xv[t][i];
            xv[t][i] *= gv[i];
          }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float4 w0 = *reinterpret_cast<const float4*>(wg + static_cast<int64_t>(e) * d + col);
        const float4 w1 = *reinterpret_cast<const float4*>(wg + static_cast<int64_t>(e) * d + col + 4);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int t = 0; t < TPB; ++t)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[t][e] = fma(static_cast<double>(xv[t][i]), static_cast<double>(wv[i]), acc[t][e]);
      }
    }
  }

  // Column sums over the 64 lanes of each wave, then over the four waves.
  double* r = red[wave];
#pragma unroll
  for (int t = 0; t < TPB; ++t) {
#pragma unroll
    for (int e = 0; e < E; ++e) r[lane * LD + t * E + e] = acc[t][e];
    if constexpr (NORM) r[lane * LD + P + t] = ss[t];
  }
  __syncthreads();
  // COLS can exceed the 64 lanes (E = 64 with the norm: 64 logits + the sum
  // of squares), so each lane reduces every 64th column.
  for (int c = lane; c < COLS; c += 64) {
    double s = 0.0;
    for (int l = 0; l < 64; ++l) s += r[l * LD + c];
    part[wave][c] = s;
  }
  __syncthreads();

  if (wave == 0) {
    const int j = lane < P ? lane : P - 1;  // idle lanes mirror the last column
    const int tl = j / E;
    const int e = j % E;
    double gd = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) gd += part[w][j];
    float g = static_cast<float>(gd);
    if constexpr (NORM) {
      double sqd = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) sqd += part[w][P + tl];
      const float sq = static_cast<float>(sqd);
      const float rinv = 1.0f / sqrtf(sq / static_cast<float>(d) + eps);
      g = static_cast<float>(gd * rinv);
      if (lane < P && e == 0) rinv_s[tl] = rinv;
    }
    if (bias != nullptr) g += bias[e];

    const int tok = tok0 + tl;
    const bool live = lane < P && tok < T;
    if (live && logits != nullptr) logits[static_cast<int64_t>(tok) * E + e] = g;

    // Top-k over the E lanes of each token: k rounds of a max butterfly
    // (larger logit first, equal logits -> lower expert index); the winner of
    // a round drops out of the next.  Then the softmax over the kept logits.
    float cand = g;
    float top_v[MAX_K];
    int top_i[MAX_K];
#pragma unroll
    for (int s = 0; s < MAX_K; ++s) {
      if (s >= k) break;
      float bv = cand;
      int bi = e;
#pragma unroll
      for (int m = E / 2; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (beats(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      top_v[s] = bv;
      top_i[s] = bi;
      if (bi == e) cand = -INFINITY;
    }
    if (live && e == 0) {
      float z = 0.f, p[MAX_K];
#pragma unroll
      for (int s = 0; s < MAX_K; ++s) {
        if (s >= k) break;
        p[s] = expf(top_v[s] - top_v[0]);
        z += p[s];
      }
      const float inv = 1.0f / z;
#pragma unroll
      for (int s = 0; s < MAX_K; ++s) {
        if (s >= k) break;
        topk_idx[static_cast<int64_t>(tok) * k + s] = top_i[s];
        topk_w[static_cast<int64_t>(tok) * k + s] = s == 0 ? 1.0f / z : p[s] * inv;
      }
    }
  }

  if constexpr (NORM) {
    // u = x * rinv * gamma for the workgroup's tokens, 8 columns per thread.
    __syncthreads();
    for (int t = 0; t < TPB && tok0 + t < T; ++t) {
      const float rt = rinv_s[t];
      for (int col = threadIdx.x * 8; col < d; col += 64 * NW * 8) {
        const int64_t off = static_cast<int64_t>(tok0 + t) * d + col;
        float xv[8];
        load_x8<XBF16>(x, off, xv);
        const float4 g0 = *reinterpret_cast<const float4*>(gamma + col);
        const float4 g1 = *reinterpret_cast<const float4*>(gamma + col + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        if constexpr (XBF16) {
          u32x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[i] = pack_bf16x2(xv[2 * i] * rt * gv[2 * i], xv[2 * i + 1] * rt * gv[2 * i + 1]);
          store16(static_cast<uint16_t*>(u_out) + off, o);
        } else {
          float4* p = reinterpret_cast<float4*>(static_cast<float*>(u_out) + off);
          p[0] = make_float4(xv[0] * rt * gv[0], xv[1] * rt * gv[1], xv[2] * rt * gv[2], xv[3] * rt * gv[3]);
          p[1] = make_float4(xv[4] * rt * gv[4], xv[5] * rt * gv[5], xv[6] * rt * gv[6], xv[7] * rt * gv[7]);
        }
      }
    }
  }
}

// Small T: one token per workgroup (T workgroups); larger T: as many tokens
// per workgroup as fit 32 logits (at most 4), so each read of the router
// weights serves several tokens and the fp64 partial sums of two workgroups
// fit one CU's LDS.  (At T = 2048 the four-token form takes 21 us against
// 33 us with the RMSNorm fused.)
constexpr int64_t kRouterOneTokenMaxT = 512;

template <int E, bool XBF16, bool NORM>
hipError_t launch_e(const void* x, const float* wg, const float* bias, const float* gamma,
                    float eps, void* u_out, float* logits, int32_t* idx, float* w, int64_t T,
                    int d, int k, hipStream_t s) {
  constexpr int TPB = (32 / E) < 1 ? 1 : ((32 / E) < 4 ? (32 / E) : 4);
  if (T <= kRouterOneTokenMaxT) {
    constexpr int NW = E <= 16 ? 8 : 4;  // fp64 transpose buffer: NW x 64 x (E + 1) doubles
    router_top2_kernel<E, 1, NW, XBF16, NORM><<<static_cast<unsigned>(T), 64 * NW, 0, s>>>(
        x, wg, bias, gamma, eps, u_out, logits, idx, w, static_cast<int>(T), d, k);
  } else {
    const dim3 grid(static_cast<unsigned>((T + TPB - 1) / TPB));
    router_top2_kernel<E, TPB, 4, XBF16, NORM><<<grid, 256, 0, s>>>(
        x, wg, bias, gamma, eps, u_out, logits, idx, w, static_cast<int>(T), d, k);
  }
  return hipGetLastError();
}

template <int E>
hipError_t launch_dtype(const void* x, bool x_bf16, const float* wg, const float* bias,
                        const float* gamma, float eps, void* u_out, float* logits, int32_t* idx,
                        float* w, int64_t T, int d, int k, hipStream_t s) {
  if (x_bf16) {
    return gamma ? launch_e<E, true, true>(x, wg, bias, gamma, eps, u_out, logits, idx, w, T, d, k, s)
                 : launch_e<E, true, false>(x, wg, bias, gamma, eps, u_out, logits, idx, w, T, d, k, s);
  }
  return gamma ? launch_e<E, false, true>(x, wg, bias, gamma, eps, u_out, logits, idx, w, T, d, k, s)
               : launch_e<E, false, false>(x, wg, bias, gamma, eps, u_out, logits, idx, w, T, d, k, s);
}

}  // namespace

hipError_t launch_route(const void* x, bool x_bf16, const float* w_gate, const float* bias,
                        float* logits, int32_t* topk_idx, float* topk_w, int64_t T, int d,
                        int E, int k, const float* gamma, float eps, void* u_out, hipStream_t stream) {
  if (k < 1 || k > MAX_K || k > E) return hipErrorInvalidValue;
  switch (E) {
    case 2: return launch_dtype<2>(x, x_bf16, w_gate, bias, gamma, eps, u_out, logits, topk_idx, topk_w, T, d, k, stream);
    case 4: return launch_dtype<4>(x, x_bf16, w_gate, bias, gamma, eps, u_out, logits, topk_idx, topk_w, T, d, k, stream);
    case 8: return launch_dtype<8>(x, x_bf16, w_gate, bias, gamma, eps, u_out, logits, topk_idx, topk_w, T, d, k, stream);
    case 16: return launch_dtype<16>(x, x_bf16, w_gate, bias, gamma, eps, u_out, logits, topk_idx, topk_w, T, d, k, stream);
    case 32: return launch_dtype<32>(x, x_bf16, w_gate, bias, gamma, eps, u_out, logits, topk_idx, topk_w, T, d, k, stream);
    case 64: return launch_dtype<64>(x, x_bf16, w_gate, bias, gamma, eps, u_out, logits, topk_idx, topk_w, T, d, k, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
