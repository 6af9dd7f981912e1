// Load-balancing loss of the router ("Mixtral" textbook page, section
// "Load-balancing loss"):
//
//   L_aux = alpha * E * sum_{s<k} sum_i f_{s,i} * P_i
//
// f_{s,i}: share of tokens whose slot-s expert (s-th largest logit) is i;
// P_i: mean over tokens of the softmax over all E router logits.  The
// statistics pool every layer's logits and every token whose mask is set.
//
// One workgroup (1024 threads, 256 for E >= 32) does the whole reduction so the result is
// bitwise deterministic: thread t takes tokens t, t + 1024, ... in order,
// selects the top-k by repeated max (larger logit first, equal logits -> lower
// index, as the router), counts slot hits with integer LDS atomics (exact,
// order-free) and accumulates its softmax sums in registers; the sums are then
// reduced by a fixed butterfly within each wave and a fixed-order sum over
// waves.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int AUX_MAX_K = 8;

template <int E, int AUX_THREADS>
__global__ __launch_bounds__(AUX_THREADS) void aux_loss_kernel(const float* __restrict__ logits, int64_t rows,
                                                               int T, int k, const uint8_t* __restrict__ mask,
                                                               float alpha, float* __restrict__ loss,
                                                               float* __restrict__ stats) {
  __shared__ int cnt[AUX_MAX_K * E];
  __shared__ float wsum[AUX_THREADS / 64][E];
  __shared__ int ntok[AUX_THREADS / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int i = tid; i < AUX_MAX_K * E; i += AUX_THREADS) cnt[i] = 0;
  __syncthreads();

  float psum[E];
#pragma unroll
  for (int e = 0; e < E; ++e) psum[e] = 0.f;
  int n = 0;
  for (int64_t r = tid; r < rows; r += AUX_THREADS) {
    if (mask != nullptr && mask[r % T] == 0) continue;
    float g[E];
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      g[e] = logits[r * E + e];
      m = fmaxf(m, g[e]);
    }
    float z = 0.f, p[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      p[e] = expf(g[e] - m);
      z += p[e];
    }
    const float inv = 1.0f / z;
#pragma unroll
    for (int e = 0; e < E; ++e) psum[e] += p[e] * inv;
    // top-k by repeated max; taken experts drop out
    uint64_t taken = 0;
    for (int s = 0; s < k; ++s) {
      int best = -1;
      float bv = -INFINITY;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool free_e = ((taken >> e) & 1ull) == 0;
        if (free_e && (best < 0 || g[e] > bv)) {
          best = e;
          bv = g[e];
        }
      }
      taken |= 1ull << best;
      atomicAdd(&cnt[s * E + best], 1);
    }
    ++n;
  }

  // Deterministic reduction of psum and n: butterfly within the wave, then
  // a fixed-order sum over the waves.
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float v = psum[e];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) wsum[wave][e] = v;
  }
  int nn = n;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) nn += __shfl_xor(nn, o, 64);
  if (lane == 0) ntok[wave] = nn;
  __syncthreads();

  if (tid == 0) {
    int N = 0;
    for (int w = 0; w < AUX_THREADS / 64; ++w) N += ntok[w];
    const float invN = N > 0 ? 1.0f / static_cast<float>(N) : 0.f;
    float acc = 0.f;
    for (int e = 0; e < E; ++e) {
      float P = 0.f;
      for (int w = 0; w < AUX_THREADS / 64; ++w) P += wsum[w][e];
      P *= invN;
      float f_tot = 0.f;
      for (int s = 0; s < k; ++s) {
        const float f = static_cast<float>(cnt[s * E + e]) * invN;
        f_tot += f;
        if (stats != nullptr) stats[s * E + e] = f;
      }
      if (stats != nullptr) stats[k * E + e] = P;
      acc += f_tot * P;
    }
    loss[0] = alpha * static_cast<float>(E) * acc;
  }
}

template <int E>
hipError_t launch_e(const float* logits, int64_t rows, int T, int k, const uint8_t* mask, float alpha, float* loss,
                    float* stats, hipStream_t s) {
  constexpr int NT = E <= 16 ? 1024 : 256;
  aux_loss_kernel<E, NT><<<1, NT, 0, s>>>(logits, rows, T, k, mask, alpha, loss, stats);
  return hipGetLastError();
}

}  // namespace

int aux_loss_max_k() { return AUX_MAX_K; }

hipError_t launch_aux_loss(const float* logits, int64_t layers, int64_t T, int E, int k, const uint8_t* mask,
                           float alpha, float* loss, float* stats, hipStream_t stream) {
  const int64_t rows = layers * T;
  const int t = static_cast<int>(T);
  switch (E) {
    case 2: return launch_e<2>(logits, rows, t, k, mask, alpha, loss, stats, stream);
    case 4: return launch_e<4>(logits, rows, t, k, mask, alpha, loss, stats, stream);
    case 8: return launch_e<8>(logits, rows, t, k, mask, alpha, loss, stats, stream);
    case 16: return launch_e<16>(logits, rows, t, k, mask, alpha, loss, stats, stream);
    case 32: return launch_e<32>(logits, rows, t, k, mask, alpha, loss, stats, stream);
    case 64: return launch_e<64>(logits, rows, t, k, mask, alpha, loss, stats, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
