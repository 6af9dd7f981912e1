// Prefill-regime expert FFN: grouped bf16 GEMM on the MFMA units.
//
//   up   (GATED): h[r]        = SiLU(x[t] W1_e^T) * (x[t] W3_e^T),  t = sorted_token[r]
//   down        : y_sorted[r] = h[r] W2_e^T
// ("Mixtral" textbook page, "Прямой проход в формулах", MoE equation, expert
// term; w1 = gate, w3 = up, w2 = down per the page's HuggingFace mapping.)
//
// Tiling.  One 512-thread workgroup computes a 256-row x 256-column tile of
// (rows of one expert) x (weight rows), K staged through LDS in 64-wide
// double-buffered slices (2 x 64 KiB).  For the up projection the 256 weight
// rows are 128 rows of W1 and the same 128 rows of W3, so the SiLU(gate) * up
// product is formed in registers and only h is written.  The eight waves sit
// 2 (rows) x 4 (columns); each computes 128 x 64 with v_mfma_f32_32x32x16_bf16
// (4 x 2 blocks of 32x32, 128 fp32 accumulators per lane), two waves per SIMD.
//
// LDS layout: row r of a [256][64] bf16 tile holds its eight 16-byte chunks
// at chunk position c ^ ((r >> 1) & 7), so the 16 consecutive rows an MFMA
// operand fetch touches fall in distinct 16-byte bank groups of the 64-bank
// LDS, and the 1 KiB a wave writes per store instruction is contiguous.
//
// Ragged expert tails.  Row tiles are numbered per expert (ceil(n_e / 256)
// each); a tile's 32-row slices past the expert's last row skip their MFMAs.
//
// Tile order.  Consecutive tile numbers walk one expert in groups of 8 column
// tiles x all of its row tiles, so blocks that share a weight tile (or an
// activation tile) are numbered, hence dispatched, together.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int BM = 256;       // rows (tokens) per tile
constexpr int BNR = 256;      // weight rows per tile
constexpr int BK = 64;        // K per LDS stage
constexpr int NTHR = 512;     // 8 waves
constexpr int NGROUP = 8;     // column tiles per tile-order group
constexpr int TILE_ELEMS = BM * BK;

__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 3); }

struct Tile {
  int e, m0, rows, n0;
};

// Tile number -> (expert, first sorted row, valid rows, first output column).
__device__ __forceinline__ bool map_tile(const int32_t* __restrict__ offsets, int E, int NT, int cols,
                                         int L, Tile& t) {
  int cum = 0;
  for (int e = 0; e < E; ++e) {
    const int lo = offsets[e];
    const int n_e = offsets[e + 1] - lo;
    const int mt = (n_e + BM - 1) / BM;
    const int cnt = mt * NT;
    if (L < cum + cnt) {
      const int i = L - cum;
      const int g = i / (mt * NGROUP);
      const int gi = i - g * mt * NGROUP;
      const int gw = min(NGROUP, NT - g * NGROUP);
      const int m = gi / gw;
      const int nn = gi - m * gw;
      t.e = e;
      t.m0 = lo + m * BM;
      t.rows = min(BM, n_e - m * BM);
      t.n0 = (g * NGROUP + nn) * cols;
      return true;
    }
    cum += cnt;
  }
  return false;
}

// Fragments of one 16-wide k-step: four 32-row A slices and two 32-row B slices.
struct Frag {
  bf16x8 a[4], b[2];
};

template <bool GATED>
__device__ __forceinline__ void read_frag(const uint16_t* As, const uint16_t* Bs, int kk, Frag& f) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2;
  const int wn = wave & 3;
  const int c = 2 * kk + (lane >> 5);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) f.a[mi] = as_bf16x8(load16(As + swz(wm * 128 + mi * 32 + (lane & 31), c)));
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int r = (GATED ? nb * 128 + wn * 32 : wn * 64 + nb * 32) + (lane & 31);
    f.b[nb] = as_bf16x8(load16(Bs + swz(r, c)));
  }
}

// FULL: every 32-row slice of the tile holds rows; otherwise slices past
// the last row (wave-uniform test) skip their MFMAs.
template <bool FULL>
__device__ __forceinline__ void mma(const Frag& f, const bool (&live)[4], f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      if (FULL || live[mi]) acc[mi][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[nb], acc[mi][nb], 0, 0, 0);
}

// Software pipeline, per 64-wide K stage kt (LDS buffer kt % 2):
//   k-step 0: store stage kt+1 (loaded one stage earlier) into the other LDS
//             buffer, issue the global loads of stage kt+2, read fragments of
//             k-step 1, MFMAs of k-step 0;
//   k-steps 1, 2: read the next k-step's fragments, MFMAs;
//   k-step 3: barrier (stage kt+1 complete in LDS, stage kt fully read), read
//             k-step 0 of stage kt+1, MFMAs of k-step 3.
template <bool GATED, bool FULL>
__device__ __forceinline__ void mainloop(const uint16_t* const (&a_src)[4], const uint16_t* const (&b_src)[4],
                                         const int (&lds_off)[4], uint16_t* sA, uint16_t* sB, int K,
                                         int rows, f32x16 (&acc)[4][2]) {
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2;
  bool live[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) live[mi] = FULL || (wm * 128 + mi * 32 < rows);

  u32x4 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = load16(a_src[i] + k0);
      rb[i] = load16(b_src[i] + k0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      store16(sA + buf * TILE_ELEMS + lds_off[i], ra[i]);
      store16(sB + buf * TILE_ELEMS + lds_off[i], rb[i]);
    }
  };

  const int KT = K / BK;
  gload(0);
  sstore(0);
  if (KT > 1) gload(1);
  __syncthreads();
  Frag f0, f1;
  read_frag<GATED>(sA, sB, 0, f0);
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const uint16_t* As = sA + cur * TILE_ELEMS;
    const uint16_t* Bs = sB + cur * TILE_ELEMS;
    // k-step 0
    if (kt + 1 < KT) sstore(cur ^ 1);
    if (kt + 2 < KT) gload(kt + 2);
    read_frag<GATED>(As, Bs, 1, f1);
    mma<FULL>(f0, live, acc);
    // k-step 1
    read_frag<GATED>(As, Bs, 2, f0);
    mma<FULL>(f1, live, acc);
    // k-step 2
    read_frag<GATED>(As, Bs, 3, f1);
    mma<FULL>(f0, live, acc);
    // k-step 3
    __syncthreads();
    if (kt + 1 < KT) read_frag<GATED>(sA + (cur ^ 1) * TILE_ELEMS, sB + (cur ^ 1) * TILE_ELEMS, 0, f0);
    mma<FULL>(f1, live, acc);
  }
}

template <bool GATED>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, void* __restrict__ out, int N, int K, int NT) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2 * TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2 * TILE_ELEMS];

  const int L = blockIdx.x;
  constexpr int COLS = GATED ? BNR / 2 : BNR;  // output columns per tile
  Tile t;
  if (!map_tile(offsets, E, NT, COLS, L, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2;
  const int wn = wave & 3;
  const int chunk = tid & 7;

  // Global->LDS copy assignment: thread copies chunk `chunk` of tile rows
  // tid/8 + 64 i of both operands.
  // Rows past the expert's last row and weight rows past N are clamped to
  // valid ones: the products they feed land in rows / columns that the
  // epilogue never stores, so the loads need no predication.
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  int lds_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 64 * i;
    const int rr = t.m0 + min(r, t.rows - 1);
    const int src = gather ? gather[rr] : rr;
    a_src[i] = A + static_cast<int64_t>(src) * K + chunk * 8;
    int n;
    const uint16_t* Bm;
    if (GATED) {
      Bm = r < 128 ? B0 : B1;
      n = t.n0 + (r & 127);
    } else {
      Bm = B0;
      n = t.n0 + r;
    }
    b_src[i] = Bm + (static_cast<int64_t>(t.e) * N + min(n, N - 1)) * K + chunk * 8;
    lds_off[i] = swz(r, chunk);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][nb][v] = 0.f;

  if (t.rows == BM)
    mainloop<GATED, true>(a_src, b_src, lds_off, sA, sB, K, t.rows, acc);
  else
    mainloop<GATED, false>(a_src, b_src, lds_off, sA, sB, K, t.rows, acc);

  // Epilogue.  32x32 accumulator layout: lane holds column lane%32 and rows
  // 8*(v/4) + 4*(lane/32) + v%4 of each 32x32 block.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 128 + mi * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= t.rows) continue;
      const int64_t row = static_cast<int64_t>(t.m0 + r) * N;
      if constexpr (GATED) {
        const int n = t.n0 + wn * 32 + (lane & 31);
        if (n < N) static_cast<uint16_t*>(out)[row + n] = f32_to_bf16(silu_fast(acc[mi][0][v]) * acc[mi][1][v]);
      } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int n = t.n0 + wn * 64 + nb * 32 + (lane & 31);
          if (n < N) static_cast<float*>(out)[row + n] = acc[mi][nb][v];
        }
      }
    }
}

template <bool GATED>
hipError_t launch(const uint16_t* A, const int32_t* gather, const int32_t* offsets, const uint16_t* B0,
                  const uint16_t* B1, void* out, int64_t rows, int N, int K, int E, hipStream_t s) {
  constexpr int COLS = GATED ? BNR / 2 : BNR;
  const int NT = (N + COLS - 1) / COLS;
  // Upper bound on the row tiles: sum_e ceil(n_e / BM) <= ceil(rows / BM) + E.
  const int64_t tiles = ((rows + BM - 1) / BM + E) * NT;
  gemm_bf16_kernel<GATED><<<static_cast<unsigned>(tiles), NTHR, 0, s>>>(A, gather, offsets, E, B0, B1, out, N, K, NT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_up_bf16(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_token,
                               const uint16_t* w1, const uint16_t* w3, uint16_t* h, int64_t T, int k, int d,
                               int d_ff, int E, hipStream_t stream) {
  return launch<true>(x, sorted_token, offsets, w1, w3, h, T * k, d_ff, d, E, stream);
}

hipError_t launch_gemm_down_bf16(const uint16_t* h, const int32_t* offsets, const uint16_t* w2, float* y_sorted,
                                 int64_t T, int k, int d, int d_ff, int E, hipStream_t stream) {
  return launch<false>(h, nullptr, offsets, w2, nullptr, y_sorted, T * k, d, d_ff, E, stream);
}

}  // namespace moe
