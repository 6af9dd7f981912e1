// Dispatch: stable counting sort of the T*k (token, slot) pairs by expert.
//
// The order is that of the expert-major algorithm on the "Mixtral" textbook
// page (section "Алгоритм"): for expert e = 0..E-1 the tokens that selected
// it, in ascending token order; empty experts get no rows.  One workgroup does the whole sort with no host round trip:
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

// Pairs a thread loads at once: its loads are independent, so a batch costs
// one memory round trip; a run of at most one batch stays in registers from
// the counting pass to the scatter.
constexpr int kDispatchBatch = 16;

template <int E, int NT>
__global__ __launch_bounds__(NT) void dispatch_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                      int k, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_token,
                                                      int32_t* __restrict__ inv_pos) {
  constexpr int B = kDispatchBatch;
  __shared__ int32_t cnt[E * NT];
  __shared__ int32_t wave_sum[NT / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = (T + NT - 1) / NT;
  // The thread's run: tokens [t0, t1), i.e. flat (token, slot) pairs [p0, p1).
  const int t0 = min(T, tid * chunk);
  const int t1 = min(T, t0 + chunk);
  const int p0 = t0 * k, p1 = t1 * k;
  int ev[B];
  auto load_batch = [&](int b) {
#pragma unroll
    for (int i = 0; i < B; ++i) ev[i] = b + i < p1 ? topk_idx[b + i] : -1;
  };

#pragma unroll
  for (int e = 0; e < E; ++e) cnt[e * NT + tid] = 0;
  for (int b = p0; b < p1; b += B) {
    load_batch(b);
    // Only this thread touches column tid of cnt; LDS atomics let the
    // increments go out back to back (the LDS applies them in order).
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int e = ev[i];
      if (e >= 0 && e < E) atomicAdd(&cnt[e * NT + tid], 1);
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

  // Scatter in the same order as the count (ev still holds a single batch).
  for (int b = p0; b < p1; b += B) {
    if (p1 - p0 > B) load_batch(b);
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int slot = b + i;
      if (slot >= p1) break;
      const int e = ev[i];
      if (e >= 0 && e < E) {
        const int pos = atomicAdd(&cnt[e * NT + tid], 1);
        sorted_token[pos] = slot / k;
        inv_pos[slot] = pos;
      } else {
        inv_pos[slot] = -1;
      }
    }
  }
}

// Many pairs: one workgroup per 256 consecutive (token, slot) pairs, so the
// scattered stores spread over many CUs.  Each workgroup first counts, over
// all pairs, those of every expert (for the expert offsets) and those before
// its own range; the row of a pair is then offsets[e] + (pairs of e before
// the range) + (pairs of e before it inside the range), the last from wave
// ballots.  Every 256-pair group lies wholly before or after a range, and
// ballots count 64 pairs per compare, so a wave counts 1024 pairs per step
// with four 16-byte loads in flight.  The rows equal the single-workgroup
// sort's (same stable order); expert counts live in scalar registers, so
// this path serves E <= 16.
constexpr int kDispatchWG = 256;  // pairs (= threads) per workgroup

template <int E>
__global__ __launch_bounds__(kDispatchWG) void dispatch_wide_kernel(const int32_t* __restrict__ topk_idx, int P,
                                                                    int k, int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ sorted_token,
                                                                    int32_t* __restrict__ inv_pos) {
  constexpr int NW = kDispatchWG / 64;
  __shared__ int32_t wtot[NW][E], wpre[NW][E], wcnt[NW][E];
  __shared__ int32_t base[E];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p_lo = blockIdx.x * kDispatchWG;
  const int p = p_lo + tid;
  const int v = p < P ? topk_idx[p] : -1;  // this thread's pair

  // 1. Counts over all pairs: wave w takes 1024-pair steps w, w + NW, ...
  int tot[E], pre[E];
#pragma unroll
  for (int e = 0; e < E; ++e) tot[e] = pre[e] = 0;
  for (int c0 = wave * 1024; c0 < P; c0 += NW * 1024) {
    int4 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i0 = c0 + 256 * j + 4 * lane;
      if (i0 + 3 < P) {
        q[j] = *reinterpret_cast<const int4*>(topk_idx + i0);
      } else {
        q[j].x = i0 < P ? topk_idx[i0] : -1;
        q[j].y = i0 + 1 < P ? topk_idx[i0 + 1] : -1;
        q[j].z = i0 + 2 < P ? topk_idx[i0 + 2] : -1;
        q[j].w = -1;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool before = c0 + 256 * j + 256 <= p_lo;  // the whole group precedes the range
      const int qv[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
      for (int e = 0; e < E; ++e) {
        int n = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) n += __popcll(__ballot(qv[c] == e));
        tot[e] += n;
        if (before) pre[e] += n;
      }
    }
  }
  // This thread's rank among the workgroup's pairs of its expert: the lanes
  // below it in its wave with the same expert, plus the earlier waves' counts.
  uint64_t mine = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t m = __ballot(v == e);
    if (v == e) mine = m;
    if (lane == 0) wcnt[wave][e] = __popcll(m);
  }
  const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mine >> 32),
                                             __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mine), 0));
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      wtot[wave][e] = tot[e];
      wpre[wave][e] = pre[e];
    }
  }
  __syncthreads();

  // 2. Expert offsets and this range's first row per expert.
  if (tid < E) {
    int off = 0, pr = 0;
    for (int e = 0; e < tid; ++e)
      for (int w = 0; w < NW; ++w) off += wtot[w][e];
    for (int w = 0; w < NW; ++w) pr += wpre[w][tid];
    base[tid] = off + pr;
    if (blockIdx.x == 0) offsets[tid] = off;
  }
  if (blockIdx.x == 0 && tid == E) {
    int all = 0;
    for (int e = 0; e < E; ++e)
      for (int w = 0; w < NW; ++w) all += wtot[w][e];
    offsets[E] = all;
  }
  __syncthreads();

  // 3. Rows.
  if (p < P) {
    if (v >= 0 && v < E) {
      int pos = base[v] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][v];
      sorted_token[pos] = p / k;
      inv_pos[p] = pos;
    } else {
      inv_pos[p] = -1;
    }
  }
}

// The wide kernel from this many pairs on.
constexpr int64_t kDispatchWideMinPairs = 2048;

template <int E>
hipError_t launch_e(const int32_t* idx, int64_t T, int k, int32_t* off, int32_t* st, int32_t* inv,
                    hipStream_t s) {
  constexpr int NT = (E <= 16) ? 1024 : (16384 / E);
  const int64_t P = T * k;
  if constexpr (E <= 16) {
    if (P >= kDispatchWideMinPairs) {
      const unsigned blocks = static_cast<unsigned>((P + kDispatchWG - 1) / kDispatchWG);
      dispatch_wide_kernel<E><<<blocks, kDispatchWG, 0, s>>>(idx, static_cast<int>(P), k, off, st, inv);
      return hipGetLastError();
    }
  }
  // Few (token, slot) pairs (decode): a single wave, whose barriers cost
  // nothing, instead of 16 waves that mostly count zeros.
  if (P <= 256)
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
