// Dispatch: stable counting sort of the T*k (token, slot) pairs by expert.
//
// The order is that of the expert-major algorithm on the "Mixtral" textbook
// page (section "Алгоритм"): for expert e = 0..E-1 the tokens that selected
// it, ascending (a row-major `where(topk_idx == e)`); empty experts get no
// rows.  One workgroup does the whole sort with no host round trip:
//   1. every thread counts its contiguous run of tokens per expert into its
//      own LDS column cnt[e][thread];
//   2. one exclusive scan over cnt in (expert, thread) order gives each
//      thread its first row per expert (expert-major, thread-minor, and the
//      threads' runs are in token order, so the result is stable);
//   3. every thread walks its run again and scatters rows.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

template <int E, int NT>
__global__ __launch_bounds__(NT) void dispatch_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                      int k, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_token,
                                                      int32_t* __restrict__ inv_pos) {
  __shared__ int32_t cnt[E * NT];
  __shared__ int32_t wave_sum[NT / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = (T + NT - 1) / NT;
  const int t0 = min(T, tid * chunk);
  const int t1 = min(T, t0 + chunk);

#pragma unroll
  for (int e = 0; e < E; ++e) cnt[e * NT + tid] = 0;
  for (int t = t0; t < t1; ++t) {
    for (int s = 0; s < k; ++s) {
      const int e = topk_idx[static_cast<int64_t>(t) * k + s];
      if (e >= 0 && e < E) cnt[e * NT + tid] += 1;
    }
  }
  __syncthreads();

  // Thread `tid` owns flat entries [tid*E, tid*E + E) of cnt (expert-major order).
  int local = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) local += cnt[tid * E + j];
  // Inclusive scan within the wave.
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += wave_sum[w];
  int run = wave_base + incl - local;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int v = cnt[tid * E + j];
    cnt[tid * E + j] = run;
    run += v;
  }
  __syncthreads();
  // First row of expert tid = its prefix at thread 0; read before the
  // scatter below starts moving the per-thread cursors.
  const int first = tid < E ? cnt[tid * NT] : 0;
  __syncthreads();
  if (tid < E) offsets[tid] = first;
  if (tid == NT - 1) offsets[E] = run;  // last thread's running total = all valid rows

  for (int t = t0; t < t1; ++t) {
    for (int s = 0; s < k; ++s) {
      const int64_t slot = static_cast<int64_t>(t) * k + s;
      const int e = topk_idx[slot];
      if (e >= 0 && e < E) {
        const int pos = cnt[e * NT + tid];
        cnt[e * NT + tid] = pos + 1;
        sorted_token[pos] = t;
        inv_pos[slot] = pos;
      } else {
        inv_pos[slot] = -1;
      }
    }
  }
}

template <int E>
hipError_t launch_e(const int32_t* idx, int64_t T, int k, int32_t* off, int32_t* st, int32_t* inv,
                    hipStream_t s) {
  constexpr int NT = (E <= 16) ? 1024 : (16384 / E);
  // Few (token, slot) pairs (decode): a single wave, whose barriers cost
  // nothing, instead of 16 waves that mostly count zeros.
  if (T * k <= 256)
    dispatch_kernel<E, 64><<<1, 64, 0, s>>>(idx, static_cast<int>(T), k, off, st, inv);
  else
    dispatch_kernel<E, NT><<<1, NT, 0, s>>>(idx, static_cast<int>(T), k, off, st, inv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const int32_t* topk_idx, int64_t T, int k, int E,
                           int32_t* expert_offsets, int32_t* sorted_token, int32_t* inv_pos,
                           hipStream_t stream) {
  switch (E) {
    case 2: return launch_e<2>(topk_idx, T, k, expert_offsets, sorted_token, inv_pos, stream);
    case 4: return launch_e<4>(topk_idx, T, k, expert_offsets, sorted_token, inv_pos, stream);
    case 8: return launch_e<8>(topk_idx, T, k, expert_offsets, sorted_token, inv_pos, stream);
    case 16: return launch_e<16>(topk_idx, T, k, expert_offsets, sorted_token, inv_pos, stream);
    case 32: return launch_e<32>(topk_idx, T, k, expert_offsets, sorted_token, inv_pos, stream);
    case 64: return launch_e<64>(topk_idx, T, k, expert_offsets, sorted_token, inv_pos, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
