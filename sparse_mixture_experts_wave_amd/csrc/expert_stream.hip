// Decode-regime expert FFN: few rows per expert, so the layer is bound by
// reading the weights.  Every touched expert's W1/W3 (up) or W2 (down) is read
// exactly once, straight from HBM into MFMA operands; experts with no rows are
// skipped, so their weights are never read.  ("Mixtral" textbook page,
// "Генерация": in generation only the selected experts run; "Прямой проход в
// формулах": the expert term (SiLU(u W_gate) * u W_up) W_down.)
//
// Work item = (touched expert, 16*NG output columns).  A workgroup of KS
// waves takes one item at a time (grid-stride over items); wave w covers the K range
// [w K/KS, (w+1) K/KS) in 128-wide steps.  With v_mfma_f32_16x16x32_bf16,
// lane (m = lane%16, q = lane/16) holds k-chunk q of each 32-wide step of
// weight row m: 64 bytes of each of 16 rows per operand register.
//
// Weight loads.  HBM streams faster (about a tenth, measured) when each load
// instruction covers whole 256-byte row segments and carries the
// non-temporal cache policy, which suits weights read exactly once (one
// M-pass covers an expert's rows whenever the streaming path is taken).  So
// each load instruction reads 4 rows x 256 bytes (buffer_load ... nt, one
// descriptor per item, all but the lane's term in the scalar offset), and the
// four loads of a 16-row step pass through a 4 KiB per-wave LDS buffer
// (16-byte chunk c of row r at slot 16 r + (c ^ r): conflict-free both ways)
// into the operand layout.
//
// The expert's rows (tokens) are the MFMA's A operand, 16 per M-block, MB
// blocks per pass.  Partial sums of the KS waves are reduced through LDS by
// wave 0, which adds the optional Linear biases ("Конфигурация", key `bias`)
// and applies the SiLU * up epilogue (up) or stores fp32 (down).
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// v[i] holds, in lane l, chunk l % 16 of row 4 i + l / 16 of a 16-row x
// 256-byte block; on return v[j] holds, in lane (m, q), chunk 4 j + q of row m.
__device__ __forceinline__ void shuffle_rows(u32x4* buf, u32x4 (&v)[4], int lane) {
  const int r = lane >> 4, c = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) buf[16 * (4 * i + r) + (c ^ (4 * i + r))] = v[i];
  const int m = lane & 15, q = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = buf[16 * m + ((4 * j + q) ^ m)];
}

// The dispatch of a decode-size layer, done by the up projection itself (no
// launch of its own): the router's top-k choices in, and the permutation the
// down projection and the combine read out.
struct FusedDispatch {
  const int32_t* topk;  // [pairs] expert of each (token, slot) pair
  int pairs, k;
  int32_t* offsets;       // [E + 1]
  int32_t* sorted_token;  // [pairs]
  int32_t* inv_pos;       // [pairs]
};
constexpr int kFuseMaxPairs = 64;
constexpr int kFuseMaxE = 64;

// With FUSED every workgroup first sorts the (token, slot) pairs by expert in
// LDS: the stable counting sort of the dispatch kernel (expert by expert,
// tokens ascending; "Mixtral" page, "Алгоритм"), at most 64 pairs, and
// workgroup 0 also stores it for the kernels that follow.
template <int MB, int NG, int KS, bool GATED, bool FUSED>
__global__ __launch_bounds__(64 * KS) void stream_ffn_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather_in,
    const int32_t* __restrict__ offsets_in, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ bias0,
    const uint16_t* __restrict__ bias1, void* __restrict__ out, int N, int K, int E, FusedDispatch fd) {
  static_assert(64 * KS > kFuseMaxE, "one thread per expert and per pair");
  __shared__ int32_t off_s[kFuseMaxE + 1];
  __shared__ int32_t row_s[kFuseMaxPairs];
  const int32_t* gather = FUSED ? row_s : gather_in;
  const int32_t* offsets = FUSED ? off_s : offsets_in;
  if constexpr (FUSED) {
    __shared__ int32_t sel[kFuseMaxPairs];
    const int tid = threadIdx.x;
    if (tid < fd.pairs) sel[tid] = fd.topk[tid];
    __syncthreads();
    if (tid < E) {
      int c = 0;
      for (int p = 0; p < fd.pairs; ++p) c += sel[p] == tid;
      off_s[tid + 1] = c;
    }
    __syncthreads();
    if (tid == 0) {
      off_s[0] = 0;
      for (int e = 0; e < E; ++e) off_s[e + 1] += off_s[e];
    }
    __syncthreads();
    if (tid < fd.pairs) {
      // Row of pair (t, s): its expert's first row plus the earlier tokens
      // that chose the same expert (a token's k experts are distinct).
      const int t = tid / fd.k, e = sel[tid];
      int rank = 0;
      for (int p = 0; p < t * fd.k; ++p) rank += sel[p] == e;
      const int pos = off_s[e] + rank;
      row_s[pos] = t;
      if (blockIdx.x == 0) {
        fd.sorted_token[pos] = t;
        fd.inv_pos[tid] = pos;
      }
    }
    if (blockIdx.x == 0 && tid <= E) fd.offsets[tid] = off_s[tid];
    __syncthreads();
  }
  constexpr int NACC = MB * NG * (GATED ? 2 : 1);
  __shared__ f32x4 red[KS - 1][NACC][64];
  // Per-wave staging of one 16-row x 256-byte weight block: row r keeps its
  // 16-byte chunk c at slot 16 r + (c ^ r), so both the row-major writes and
  // the operand-layout reads touch 16 distinct bank groups per 16 lanes.
  __shared__ u32x4 shuf[KS][256];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15;
  const int q = lane >> 4;
  const int Kw = K / KS;
  const int kb = wave * Kw;
  const int tiles = N / (16 * NG);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // Work items cover only the experts that received rows, so all workgroups
  // share the touched experts' weights however few they are.
  int touched = 0;
  for (int e = 0; e < E; ++e) touched += offsets[e + 1] > offsets[e];
  const int items = touched * tiles;

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int j = item / tiles;  // j-th touched expert
    int e = 0;
    for (int seen = -1; e < E; ++e) {
      seen += offsets[e + 1] > offsets[e];
      if (seen == j) break;
    }
    const int n0 = (item - j * tiles) * (16 * NG);
    const int lo = offsets[e];
    const int n_e = offsets[e + 1] - lo;

    // Weight loads: four rows x 256 bytes per instruction (lane l: row
    // l / 16 of the instruction's four, bytes 16 (l % 16)), through a buffer
    // descriptor at the item's first weight row; every per-load term but the
    // lane's goes into the scalar offset.
    const int64_t row0 = static_cast<int64_t>(e) * N + n0;
    const __amdgpu_buffer_rsrc_t rs0 = wave_rsrc(B0 + row0 * K);
    const __amdgpu_buffer_rsrc_t rs1 = GATED ? wave_rsrc(B1 + row0 * K) : rs0;
    const uint32_t lane_off = static_cast<uint32_t>((lane >> 4) * K + 8 * (lane & 15)) * 2u;

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
          for (int i = 0; i < 4; ++i) {
            const int soff = ((16 * g + 4 * i) * K + kb + k) * 2;
            w0[g][i] = load16_buf_nt(rs0, lane_off, soff);
            if constexpr (GATED) w1[g][i] = load16_buf_nt(rs1, lane_off, soff);
          }
        // Into the operand layout: lane (m, q) needs row m, chunk 4 j + q.
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          shuffle_rows(shuf[wave], w0[g], lane);
          if constexpr (GATED) shuffle_rows(shuf[wave], w1[g], lane);
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
                acc1[mb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[mb][j]),
                                                                      as_bf16x8(w1[g][j]), acc1[mb][g], 0, 0, 0);
            }
      }

      // Reduce the KS partial sums through LDS into wave 0.
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
        for (int w = 0; w < KS - 1; ++w) {
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
        float bb0[NG], bb1[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int64_t bi = static_cast<int64_t>(e) * N + n0 + 16 * g + m;
          bb0[g] = bias0 ? bf16_to_f32(bias0[bi]) : 0.f;
          bb1[g] = (GATED && bias1) ? bf16_to_f32(bias1[bi]) : 0.f;
        }
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
                  static_cast<uint16_t*>(out)[o] =
                      f32_to_bf16(silu_fast(acc0[mb][g][v] + bb0[g]) * (acc1[mb][g][v] + bb1[g]));
                else
                  static_cast<float*>(out)[o] = acc0[mb][g][v] + bb0[g];
              }
            }
      }
      __syncthreads();
    }
  }
}

// Weights, biases and output of one projection.
struct Proj {
  const uint16_t* B0;
  const uint16_t* B1;
  const uint16_t* bias0;
  const uint16_t* bias1;
  void* out;
};

template <int MB, int NG, int KS, bool GATED, bool FUSED = false>
hipError_t launch_cfg(const uint16_t* A, const int32_t* gather, const int32_t* offsets, const Proj& p, int N,
                      int K, int E, int grid, hipStream_t s, const FusedDispatch& fd = {}) {
  const int items = E * (N / (16 * NG));
  const int blocks = grid > 0 && grid < items ? grid : items;
  stream_ffn_bf16_kernel<MB, NG, KS, GATED, FUSED><<<blocks, 64 * KS, 0, s>>>(
      A, gather, offsets, p.B0, p.B1, p.bias0, p.bias1, p.out, N, K, E, fd);
  return hipGetLastError();
}

template <int NG, int KS, bool GATED, bool FUSED = false>
hipError_t launch_mb(int64_t T, const uint16_t* A, const int32_t* gather, const int32_t* offsets, const Proj& p,
                     int N, int K, int E, int grid, hipStream_t s, const FusedDispatch& fd = {}) {
  // n_e <= T: the experts of one token are distinct.
  if (T <= 16) return launch_cfg<1, NG, KS, GATED, FUSED>(A, gather, offsets, p, N, K, E, grid, s, fd);
  if (T <= 32) return launch_cfg<2, NG, KS, GATED, FUSED>(A, gather, offsets, p, N, K, E, grid, s, fd);
  return launch_cfg<4, NG, KS, GATED, FUSED>(A, gather, offsets, p, N, K, E, grid, s, fd);
}

// Workgroups of the grid-stride loop (8 per CU on 256 CUs): enough bytes in
// flight to saturate HBM, without a ragged last round of one-item workgroups.
constexpr int kStreamGrid = 2048;

}  // namespace

bool stream_supported(int64_t T, int d, int d_ff) {
  return T <= kStreamMaxT && d % 512 == 0 && d_ff % 512 == 0;
}

hipError_t launch_stream_up_bf16(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_token,
                                 const uint16_t* w1, const uint16_t* w3, const uint16_t* b1,
                                 const uint16_t* b3, uint16_t* h, int64_t T, int d, int d_ff, int E,
                                 hipStream_t stream) {
  const Proj p{w1, w3, b1, b3, h};
  // Few tokens touch few experts (up to about 7 at T = 8): narrower work
  // items (16 columns) keep every workgroup busy; the K split doubles when it
  // divides evenly.
  if (T <= 8 && d % 1024 == 0)  // at most 8 rows per expert: one 16-row M-block
    return launch_cfg<1, 1, 8, true>(x, sorted_token, offsets, p, d_ff, d, E, kStreamGrid, stream);
  return launch_mb<2, 4, true>(T, x, sorted_token, offsets, p, d_ff, d, E, kStreamGrid, stream);
}

bool stream_dispatch_supported(int64_t T, int k, int d, int d_ff, int E) {
  return stream_supported(T, d, d_ff) && T * k <= kFuseMaxPairs && E <= kFuseMaxE;
}

hipError_t launch_stream_up_dispatch_bf16(const uint16_t* x, const int32_t* topk_idx, int k, int32_t* offsets,
                                          int32_t* sorted_token, int32_t* inv_pos, const uint16_t* w1,
                                          const uint16_t* w3, const uint16_t* b1, const uint16_t* b3, uint16_t* h,
                                          int64_t T, int d, int d_ff, int E, hipStream_t stream) {
  if (!stream_dispatch_supported(T, k, d, d_ff, E)) return hipErrorInvalidValue;
  const Proj p{w1, w3, b1, b3, h};
  const FusedDispatch fd{topk_idx, static_cast<int>(T) * k, k, offsets, sorted_token, inv_pos};
  // The same configurations as launch_stream_up_bf16.
  if (T <= 8 && d % 1024 == 0)
    return launch_cfg<1, 1, 8, true, true>(x, nullptr, nullptr, p, d_ff, d, E, kStreamGrid, stream, fd);
  return launch_mb<2, 4, true, true>(T, x, nullptr, nullptr, p, d_ff, d, E, kStreamGrid, stream, fd);
}

hipError_t launch_stream_down_bf16(const uint16_t* h, const int32_t* offsets, const uint16_t* w2,
                                   const uint16_t* b2, float* y_sorted, int64_t T, int d, int d_ff, int E,
                                   hipStream_t stream) {
  const Proj p{w2, nullptr, b2, nullptr, y_sorted};
  // With 1-8 tokens only 2-7 experts are touched: an 8-way K split keeps
  // enough loads in flight when it divides evenly (at T = 8 it takes the
  // layer from 399 to 386 us).
  if (T <= 8 && d_ff % 1024 == 0)  // one 16-row M-block, as above
    return launch_cfg<1, 1, 8, false>(h, nullptr, offsets, p, d, d_ff, E, kStreamGrid, stream);
  if (T <= 4) return launch_cfg<1, 1, 4, false>(h, nullptr, offsets, p, d, d_ff, E, kStreamGrid, stream);
  // Up to 16 tokens: 64-column items, so each step's weight loads (16 KiB per
  // wave) outweigh its activation loads 4 : 1 (0.7 % faster than 32 columns
  // at T = 16).
  if (T <= 16) return launch_cfg<1, 4, 4, false>(h, nullptr, offsets, p, d, d_ff, E, kStreamGrid, stream);
  return launch_mb<2, 4, false>(T, h, nullptr, offsets, p, d, d_ff, E, kStreamGrid, stream);
}

}  // namespace moe
