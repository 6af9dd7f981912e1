// Prefill-regime expert FFN: grouped bf16 GEMM on the MFMA units.
//
//   up   (GATED): h[r]        = SiLU(x[t] W1_e^T + b1_e) * (x[t] W3_e^T + b3_e),  t = sorted_token[r]
//   down        : y_sorted[r] = h[r] W2_e^T + b2_e
// ("Mixtral" textbook page, "Прямой проход в формулах", MoE equation, expert
// term; w1 = gate, w3 = up, w2 = down per the page's HuggingFace mapping; the
// Linear biases are optional, section "Конфигурация", key `bias`.)
//
// Tiling.  One 512-thread workgroup computes a 256-row x 256-column tile of
// (rows of one expert) x (weight rows).  For the up projection the 256 weight
// rows are 128 rows of W1 and the same 128 rows of W3, so SiLU(gate) * up is
// formed in registers and only h is written.  The eight waves sit 2 (rows) x 4
// (columns); each computes 128 x 64 with v_mfma_f32_16x16x32_bf16 (8 x 4
// blocks of 16x16, one MFMA per block and 32-wide K slice, 128 fp32
// accumulators per lane).  Under sustained load the chip is power-limited,
// and 16x16x32 MFMAs run at a higher clock than 32x32x16 ones for the same
// work (all CUs, random bf16 operands: 2.02-2.05 against 1.73-1.80 GHz).  In
// this kernel that raises the clock from 1.53 to 1.72 GHz but the matrix
// cores then wait more (busy 0.64 against 0.73): the tile's throughput is set
// by the global -> LDS copies, not by the MFMA rate; the 16x16 blocks cost
// fewer registers and speed up the down projection a little.
//
// Ping-pong schedule.  Waves 0-3 (group 0) and 4-7 (group 1) put one wave of
// each group on every SIMD, and the groups run half a step apart: while one
// group issues the 32 MFMAs of a 32-wide K slice, the other reads its next
// slice's operands from LDS and issues its share of the global -> LDS copies.
// Every such interval ends in a barrier of all eight waves, so the matrix core
// of each SIMD always has one wave feeding it.  Group 0 copies the A slices,
// group 1 the B slices.
//
// Data movement.  K is staged in 32-wide slices through a ring of NS = 5 LDS
// slots (5 x 32 KiB, all of the CU's LDS).  Copies go straight from memory to
// LDS (buffer_load_dwordx4 ... lds: no staging registers, no LDS store
// instructions) through one buffer descriptor per wave.  A copy instruction
// moves 16 rows x 64 bytes; slices 2m and 2m+1 are the two halves of the same
// 128-byte row segments, so they are copied in pairs, back to back per row
// group, which costs the memory pipeline about a quarter less than copying
// each slice on its own.  Half of a pair goes out in each of two consecutive
// memory phases, into the slots of slices that were read at least one
// interval before, and each wave waits for its own copies of slice s+1
// (s_waitcnt vmcnt) just before the barrier that opens it.
// The main loop runs ten slices per trip and each wave group its own copy of
// it, so every step's ring slot, copy parity and LDS destinations are
// compile-time constants; copies past the last slice re-copy the last one
// into a slot no wave still reads, which keeps every wait count constant
// (about 5 % faster than runtime slot parity and guarded copies).
//
// LDS layout: a slice is [256 rows][32] bf16, 64 bytes per row; row r keeps
// its four 16-byte chunks at position c ^ ((r >> 2) & 3), so the 16
// consecutive rows that one operand read touches land in 16 distinct 16-byte
// bank groups of the 64-bank LDS.  A copy instruction writes 1 KiB (16 rows)
// contiguously; each lane picks the global chunk that belongs at its slot.
//
// Ragged expert tails.  Row tiles are numbered per expert (ceil(n_e / 256)
// each); a tile's 16-row blocks past the expert's last row skip their MFMAs.
// Rows past the last one (and weight rows past N) are clamped to valid rows:
// their products land in rows / columns the epilogue never stores.
//
// Tile order.  Consecutive tile numbers walk one expert in groups of 8 column
// tiles x 4 row tiles, row tile by row tile within a group, so blocks that
// share a weight tile (or an activation tile) are numbered together.
// Workgroups go to the 8 XCDs (each with its own L2) in turn, so an XCD gets
// one column of each group: while a round of 256 runs, each XCD holds 8 weight
// tiles and 4 activation tiles, each used 4 and 8 times.  (Groups of all of a
// large expert's row tiles would give an XCD one weight tile and 32 activation
// tiles, fetched again by every XCD and every column group.)
//
// The last round.  A workgroup fills a CU (all of its LDS), so tiles run in
// rounds of one per CU; when the tile count is not a multiple of the CU count
// the last round would leave CUs idle (the down projection at T = 4096 has
// 2 full rounds and 48 tiles).  Given a partial-sum buffer, the R tiles of the
// last round are each split along K into S = floor(CUs / R) pieces (whole
// slice pairs, at most 8); a piece stores its fp32 accumulators, and a fix-up
// kernel adds a tile's S partial sums in piece order (deterministic) and runs
// the same epilogue.
#include "device_common.h"
#include "kernels.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int BM = 256;    // rows (tokens) per tile
constexpr int BNR = 256;   // weight rows per tile
constexpr int BK = 32;     // K per LDS slice
constexpr int NS = 5;      // LDS ring depth (slices)
constexpr int NTHR = 512;  // 8 waves
constexpr int NGROUP = 8;  // column tiles per tile-order group
constexpr int RBLOCK = 4;  // row tiles per tile-order group
constexpr int SLICE = BM * BK;  // elements per operand slice
constexpr int COPIES = 4;       // copy instructions per thread per slice
constexpr int MAX_SPLIT = 8;    // K pieces per split tile
constexpr int ACC_CHUNKS = 32;  // float4 chunks of one thread's 128 accumulators

static_assert(2 * NS * SLICE * 2 <= 163840, "LDS ring exceeds 160 KiB");

__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ ((r >> 2) & 3)) << 3); }

// s_waitcnt with only a vmcnt limit (expcnt, lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}
// s_waitcnt with only an lgkmcnt limit (vmcnt, expcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(N >= 0 && N < 16, "lgkmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
}

// A barrier that the compiler may move no instruction across, LDS accesses
// included: the s_barrier builtin is not a memory barrier for the optimizer,
// which could otherwise hoist an operand read above the barrier that
// publishes its slice.  No wait is emitted: each wave has already waited
// (s_waitcnt) for the copies it publishes.
__device__ __forceinline__ void bar() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// The barriers that only one wave group executes (the half-step offset) carry
// asm text of their own: the optimiser never executes a volatile asm on a
// path where it was not, but it may merge identical ones, and merging one of
// these with a barrier both groups run would change the barrier counts.
__device__ __forceinline__ void bar_group1_start() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier  ; group 1 starts one interval late" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void bar_group0_end() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier  ; group 0 ends one interval late" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

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
      const int rb = i / (RBLOCK * NT);          // row block (the last may be short)
      const int rbr = min(RBLOCK, mt - rb * RBLOCK);
      const int ib = i - rb * RBLOCK * NT;
      const int g = ib / (rbr * NGROUP);
      const int gi = ib - g * rbr * NGROUP;
      const int gw = min(NGROUP, NT - g * NGROUP);
      const int m = rb * RBLOCK + gi / gw;
      const int nn = gi - (gi / gw) * gw;
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

// Operands of one 32-wide K slice: eight 16-row A blocks and four 16-row B
// blocks.  With v_mfma_f32_16x16x32_bf16, lane (r = lane % 16, c = lane / 16)
// holds the 16-byte chunk c (k = 8c .. 8c+7) of row r of each block.
struct Frag {
  bf16x8 a[8], b[4];
};

// Weight row (within the tile) of B block nb's row r.  Gated: blocks 0, 1 are
// W1 rows (gate) and 2, 3 the same rows of W3 (up).
template <bool GATED>
__device__ __forceinline__ int b_row(int wn, int nb, int r) {
  return (GATED ? (nb >> 1) * 128 + wn * 32 + (nb & 1) * 16 : wn * 64 + nb * 16) + r;
}

template <bool GATED>
__device__ __forceinline__ void read_frag(const uint16_t* As, const uint16_t* Bs, Frag& f) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2;
  const int wn = wave & 3;
  const int c = lane >> 4, r = lane & 15;
  // A blocks 0, 1, 4, 5 first: they hold rows 0-31 of each wave's 64-row
  // copy block, the rows a copy may reach one interval later (see slice_step).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mi = (i & 1) + 4 * (i >> 1);
    f.a[mi] = as_bf16x8(load16(As + swz(wm * 128 + mi * 16 + r, c)));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mi = 2 + (i & 1) + 4 * (i >> 1);
    f.a[mi] = as_bf16x8(load16(As + swz(wm * 128 + mi * 16 + r, c)));
  }
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) f.b[nb] = as_bf16x8(load16(Bs + swz(b_row<GATED>(wn, nb, r), c)));
}

// FULL: every 16-row block of the tile is multiplied; otherwise blocks past
// the last row (a wave-uniform test) skip their MFMAs.
template <bool FULL>
__device__ __forceinline__ void mma(const Frag& f, const bool (&live)[8], f32x4 (&acc)[8][4]) {
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      if (FULL || live[mi]) acc[mi][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[mi], f.b[nb], acc[mi][nb], 0, 0, 0);
}

// The LDS ring: NS slices of A and of B, each a distinct array, so that the
// compiler can tell a copy into one slot from an operand read of another
// (slot indices below are compile-time constants).
__shared__ __attribute__((aligned(1024))) uint16_t lds_a0[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_a1[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_a2[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_a3[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_a4[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_b0[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_b1[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_b2[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_b3[SLICE];
__shared__ __attribute__((aligned(1024))) uint16_t lds_b4[SLICE];

template <int B>
__device__ __forceinline__ uint16_t* ring_a() {
  static_assert(B >= 0 && B < NS, "slot");
  if constexpr (B == 0) return lds_a0;
  else if constexpr (B == 1) return lds_a1;
  else if constexpr (B == 2) return lds_a2;
  else if constexpr (B == 3) return lds_a3;
  else return lds_a4;
}
template <int B>
__device__ __forceinline__ uint16_t* ring_b() {
  static_assert(B >= 0 && B < NS, "slot");
  if constexpr (B == 0) return lds_b0;
  else if constexpr (B == 1) return lds_b1;
  else if constexpr (B == 2) return lds_b2;
  else if constexpr (B == 3) return lds_b3;
  else return lds_b4;
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Where this thread's copies come from: the wave's buffer descriptor and the
// byte offset of each of its four 16-byte chunks at K = 0.
struct CopySrc {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[COPIES];
  int last;  // the last K slice of the tile (or piece)
  int woff;  // element offset of the wave's first row (64 (w & 3)) in a slot
};

// One copy: row group j (rows 64 (w & 3) + 16 j + lane / 4) of K slice s into
// ring slot B; group 0 copies A, group 1 copies B (GRP is the wave's group).
// A slice past the last one is copied as the last one: the schedule stays the
// same to the end, and such a copy lands in the slot of a slice every wave
// has finished with.
template <int B, int GRP>
__device__ __forceinline__ void copy_one(const CopySrc& cs, int s, int j) {
  uint16_t* ring = GRP == 0 ? ring_a<B>() : ring_b<B>();
  __builtin_amdgcn_raw_ptr_buffer_load_lds(cs.rsrc, (lds_ptr)(ring + cs.woff + j * 16 * BK), 16,
                                           cs.off[j] + min(s, cs.last) * (BK * 2), 0, 0, 0);
}

// Slices 2m and 2m+1 hold the two 64-byte halves of the same 128-byte row
// segments, so their copies go out in pairs, back to back per row group:
// the second copy of a pair reads lines the first has just brought in.  Row
// groups j0, j0+1 of the pair (s0, s0+1) into slots SA, SB.
template <int SA, int SB, int GRP>
__device__ __forceinline__ void copy_pair_half(const CopySrc& cs, int s0, int j0) {
#pragma unroll
  for (int j = j0; j < j0 + 2; ++j) {
    copy_one<SA, GRP>(cs, s0, j);
    copy_one<SB, GRP>(cs, s0 + 1, j);
  }
}

// Issue schedule: the memory phase of an odd slice s copies row groups 0, 1
// of the pair (s+3, s+4); that of an even slice s copies row groups 2, 3 of
// the pair (s+2, s+3).  Before the barrier that opens slice s+1, each wave
// waits for its own copies of s+1: 5 younger copies may stay in flight after
// an odd slice, 8 after an even one.
template <bool ODD>
__device__ __forceinline__ void wait_slice_next() {
  if constexpr (ODD) wait_vmcnt<5>();
  else wait_vmcnt<8>();
}

// One K slice s (ring slot B = s % NS, ODD = s & 1, both fixed at compile
// time), as two intervals: memory phase (operand reads of slice s, half a
// pair of copies) and compute phase (32 MFMAs).  Group 1 runs each phase one
// interval after group 0.
//
// Operand reads land in the wave's own registers and the MFMAs of the next
// interval wait for each one (lgkmcnt) as they need it, so a memory phase
// waits for its reads before the barrier only where a copy could overwrite
// them in the very next interval.  The next copy into slot B is that of
// slice s+5: group 0 issues half of it (A, rows 0-31 of each 64-row copy
// block) at its odd step s+1 when s is even, one interval after group 1 has
// read slice s; every other one comes two or more intervals after the reads,
// by when the reading wave's own MFMAs have waited for them.  So group 1
// waits at even steps only, and only for its A reads of those rows (blocks
// 0, 1, 4, 5, issued first: lgkmcnt(8) leaves the other eight reads in
// flight).  (Waiting for every read in every memory phase kept the group from
// the barrier for the reads' whole latency: 4-5 % of the kernel.)
template <bool GATED, bool FULL, int GRP, int B, bool ODD>
__device__ __forceinline__ void slice_step(const CopySrc& cs, int s, const bool (&live)[8], f32x4 (&acc)[8][4]) {
  Frag f;
  read_frag<GATED>(ring_a<B>(), ring_b<B>(), f);
  if constexpr (ODD)
    copy_pair_half<(B + 3) % NS, (B + 4) % NS, GRP>(cs, s + 3, 0);
  else
    copy_pair_half<(B + 2) % NS, (B + 3) % NS, GRP>(cs, s + 2, 2);
  if constexpr (GRP == 1 && !ODD) {
    __builtin_amdgcn_sched_barrier(0);  // all twelve reads issued before the count is taken
    wait_lgkm<8>();                     // the four reads issued first have landed
  }
  if constexpr (GRP == 1) wait_slice_next<ODD>();
  bar();
  mma<FULL>(f, live, acc);
  if constexpr (GRP == 0) wait_slice_next<ODD>();
  bar();
}

template <bool GATED, bool FULL, int GRP>
__device__ __forceinline__ void mainloop_grp(CopySrc& cs, int K, int rows, f32x4 (&acc)[8][4]) {
  bool live[8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) live[mi] = FULL || (GRP * 128 + mi * 16 < rows);

  const int KT = K / BK;  // >= 2 and even (K is a multiple of 64)
  cs.last = KT - 1;
  // Prologue: slices 0 and 1 whole, row groups 0, 1 of slices 2 and 3.
  copy_pair_half<0, 1, GRP>(cs, 0, 0);
  copy_pair_half<0, 1, GRP>(cs, 0, 2);
  copy_pair_half<2, 3, GRP>(cs, 2, 0);
  wait_vmcnt<5>();  // slice 0's last copy is followed by 5
  bar();
  if constexpr (GRP == 1) bar_group1_start();
  // Ten slices per trip, so that each step's ring slot and parity are fixed.
  int s = 0;
  for (; s + 2 * NS <= KT; s += 2 * NS) {
    slice_step<GATED, FULL, GRP, 0, false>(cs, s, live, acc);
    slice_step<GATED, FULL, GRP, 1, true>(cs, s + 1, live, acc);
    slice_step<GATED, FULL, GRP, 2, false>(cs, s + 2, live, acc);
    slice_step<GATED, FULL, GRP, 3, true>(cs, s + 3, live, acc);
    slice_step<GATED, FULL, GRP, 4, false>(cs, s + 4, live, acc);
    slice_step<GATED, FULL, GRP, 0, true>(cs, s + 5, live, acc);
    slice_step<GATED, FULL, GRP, 1, false>(cs, s + 6, live, acc);
    slice_step<GATED, FULL, GRP, 2, true>(cs, s + 7, live, acc);
    slice_step<GATED, FULL, GRP, 3, false>(cs, s + 8, live, acc);
    slice_step<GATED, FULL, GRP, 4, true>(cs, s + 9, live, acc);
  }
  // The rest: an even number of slices below ten (s is a multiple of 10).
  if (s < KT) {
    slice_step<GATED, FULL, GRP, 0, false>(cs, s, live, acc);
    slice_step<GATED, FULL, GRP, 1, true>(cs, s + 1, live, acc);
  }
  if (s + 2 < KT) {
    slice_step<GATED, FULL, GRP, 2, false>(cs, s + 2, live, acc);
    slice_step<GATED, FULL, GRP, 3, true>(cs, s + 3, live, acc);
  }
  if (s + 4 < KT) {
    slice_step<GATED, FULL, GRP, 4, false>(cs, s + 4, live, acc);
    slice_step<GATED, FULL, GRP, 0, true>(cs, s + 5, live, acc);
  }
  if (s + 6 < KT) {
    slice_step<GATED, FULL, GRP, 1, false>(cs, s + 6, live, acc);
    slice_step<GATED, FULL, GRP, 2, true>(cs, s + 7, live, acc);
  }
  if constexpr (GRP == 0) bar_group0_end();  // same barrier count for both groups
  wait_vmcnt<0>();  // the copies issued past the last slice land before the workgroup's LDS is released
}

template <bool GATED, bool FULL>
__device__ __forceinline__ void mainloop(CopySrc& cs, int K, int rows, f32x4 (&acc)[8][4]) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  cs.woff = (wave & 3) * 64 * BK;
  if (wave < 4)
    mainloop_grp<GATED, FULL, 0>(cs, K, rows, acc);
  else
    mainloop_grp<GATED, FULL, 1>(cs, K, rows, acc);
}

// Number of tiles (sum over experts of the row tiles, times NT).
__device__ __forceinline__ int count_tiles(const int32_t* __restrict__ offsets, int E, int NT) {
  int total = 0;
  for (int e = 0; e < E; ++e) total += (offsets[e + 1] - offsets[e] + BM - 1) / BM * NT;
  return total;
}

// Which tiles run whole and which are split: tiles [0, full) whole, the R
// tiles after them in S pieces each (S = 1: none split).
struct SplitPlan {
  int full, R, S;
};

__device__ __forceinline__ SplitPlan split_plan(int total, int cus, int KT, bool can_split) {
  SplitPlan p;
  p.full = total / cus * cus;
  p.R = total - p.full;
  p.S = 1;
  if (can_split && p.R > 0) p.S = min(min(cus / p.R, MAX_SPLIT), KT / 4);
  if (p.S < 2) {
    p.S = 1;
    p.full = total;
    p.R = 0;
  }
  return p;
}

// Destination of the fused Q|K|V projection of attention, with RoPE: of the N
// output columns, [0, nq) go to q, [nq, nq + nkv) to k, the rest to v, each a
// bf16 row-major [rows][width] matrix.  In q and k the pair of columns
// (2i, 2i+1) of each 128-wide head is turned by the angle whose cosine and
// sine are cs[row][i] (x0, x1 -> x0 c - x1 s, x0 s + x1 c).  q == nullptr:
// not this epilogue.
struct RopeOut {
  uint16_t* q;
  uint16_t* k;
  uint16_t* v;
  const float2* cs;  // [rows][64]
  int nq, nkv;
};

// The value of the neighbouring lane of the pair (lane ^ 1): columns 2i and
// 2i+1 of one row sit in adjacent lanes of the accumulator layout.
__device__ __forceinline__ float swap_pair(float y) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), 0xB1, 0xF, 0xF, false));
}

// Epilogue of one tile: biases, then SiLU(gate) * up rounded to bf16 (up) or
// fp32 (down).  16x16 accumulator layout: lane holds column lane%16 and rows
// 4*(lane/16) + v of each 16x16 block.  Gated: blocks nb and nb + 2 hold the
// gate and up sums of the same output column.
// Only the rows of 32-row blocks [mlo, mhi) of each wave (16-row blocks
// [2 mlo, 2 mhi)) are stored.  With resid set (not gated) the fp32 result is
// not stored: it is added to the bf16 matrix resid in place with one
// rounding, resid = bf16(resid + (acc + bias)), the residual connection after
// an output projection.  With ro.q set (not gated) the result goes to q, k, v
// as RopeOut describes.
template <bool GATED>
__device__ __forceinline__ void store_tile(const Tile& t, const f32x4 (&acc)[8][4],
                                           const uint16_t* __restrict__ bias0,
                                           const uint16_t* __restrict__ bias1, void* __restrict__ out,
                                           uint16_t* __restrict__ resid, const RopeOut& ro, int N,
                                           int mlo = 0, int mhi = 4) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2;
  const int wn = wave & 3;
  const int lc = lane & 15, lr = 4 * (lane >> 4);  // the lane's column and first row in a block
  // Output column of block nb (gated: of blocks nb and nb + 2).
  auto col = [&](int nb) { return GATED ? t.n0 + wn * 32 + (nb & 1) * 16 + lc : t.n0 + wn * 64 + nb * 16 + lc; };
  float bb[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = col(nb);
    const uint16_t* bsrc = (GATED && nb >= 2) ? bias1 : bias0;
    bb[nb] = (bsrc && n < N) ? bf16_to_f32(bsrc[static_cast<int64_t>(t.e) * N + n]) : 0.f;
  }
  if constexpr (!GATED) {
    if (ro.q) {
      // The wave's 64 columns lie in one 128-wide head (N, nq and nkv are
      // multiples of 128), so the destination is wave-uniform.
      const int nw = t.n0 + wn * 64;
      if (nw >= N) return;
      uint16_t* dst = ro.v;
      int ld = ro.nkv, c0 = nw - ro.nq - ro.nkv;
      bool rot = false;
      if (nw < ro.nq) {
        dst = ro.q, ld = ro.nq, c0 = nw, rot = true;
      } else if (nw < ro.nq + ro.nkv) {
        dst = ro.k, ld = ro.nkv, c0 = nw - ro.nq, rot = true;
      }
      const bool odd = lane & 1;
      const int i0 = ((c0 & 127) + lc) >> 1;  // pair index of block nb = 0; block nb adds 8 nb
#pragma unroll
      for (int mi = 0; mi < 8; ++mi) {
        if (mi < 2 * mlo || mi >= 2 * mhi) continue;
        // The block's angles first (rows clamped into the tile, as for the
        // residual loads), so that their loads overlap.
        float2 cs[4][4];
        if (rot) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const int r = min(wm * 128 + mi * 16 + lr + v, t.rows - 1);
              cs[v][nb] = ro.cs[static_cast<int64_t>(t.m0 + r) * 64 + i0 + 8 * nb];
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int r = wm * 128 + mi * 16 + lr + v;
            float y = acc[mi][nb][v] + bb[nb];
            if (rot) {
              // Both lanes of a pair hold the same row, so they take this
              // branch and the swap together.
              const float p = swap_pair(y);
              const float x0 = odd ? p : y, x1 = odd ? y : p;
              const float c = cs[v][nb].x, sn = cs[v][nb].y;
              y = odd ? x0 * sn + x1 * c : x0 * c - x1 * sn;
            }
            if (r < t.rows) dst[static_cast<int64_t>(t.m0 + r) * ld + c0 + nb * 16 + lc] = f32_to_bf16(y);
          }
      }
      return;
    }
    if (resid) {
      // Per 16-row block: every residual load is issued before the first
      // store, so their latencies overlap.  The loads are unconditional (rows
      // and columns past the tile's edge are clamped to its last valid one)
      // so that no branch forces a wait between them.
#pragma unroll
      for (int mi = 0; mi < 8; ++mi) {
        if (mi < 2 * mlo || mi >= 2 * mhi) continue;
        uint16_t hv[4][4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int r = min(wm * 128 + mi * 16 + lr + v, t.rows - 1);
            const int n = min(col(nb), N - 1);
            hv[v][nb] = resid[static_cast<int64_t>(t.m0 + r) * N + n];
          }
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int r = wm * 128 + mi * 16 + lr + v;
            const int n = col(nb);
            if (r < t.rows && n < N)
              resid[static_cast<int64_t>(t.m0 + r) * N + n] =
                  f32_to_bf16(bf16_to_f32(hv[v][nb]) + (acc[mi][nb][v] + bb[nb]));
          }
      }
      return;
    }
  }
  // The plain outputs.  The epilogue runs on every wave at once, after the
  // main loop, so its vector instruction count is time the matrix cores
  // stand idle: without biases the adds are left out, and the gated outputs
  // are rounded two at a time (v_cvt_pk_bf16_f32, round to nearest even like
  // f32_to_bf16) and stored from the halves of the packed word.
  const bool has_bias = bias0 != nullptr || (GATED && bias1 != nullptr);
  auto plain = [&](auto with_bias) {
    constexpr bool B = decltype(with_bias)::value;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      if (mi < 2 * mlo || mi >= 2 * mhi) continue;
      const int r0 = wm * 128 + mi * 16 + lr;  // rows r0 .. r0 + 3
      if constexpr (GATED) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int n = col(nb);
          float y[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float g = B ? acc[mi][nb][v] + bb[nb] : acc[mi][nb][v];
            const float u = B ? acc[mi][nb + 2][v] + bb[nb + 2] : acc[mi][nb + 2][v];
            y[v] = silu_fast(g) * u;
          }
          const uint32_t p01 = cvt_pk_bf16(y[0], y[1]), p23 = cvt_pk_bf16(y[2], y[3]);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t p = v < 2 ? p01 : p23;
            if (r0 + v < t.rows && n < N)
              static_cast<uint16_t*>(out)[static_cast<int64_t>(t.m0 + r0 + v) * N + n] =
                  static_cast<uint16_t>((v & 1) ? p >> 16 : p);
          }
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (r0 + v >= t.rows) continue;
          const int64_t row = static_cast<int64_t>(t.m0 + r0 + v) * N;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int n = col(nb);
            if (n < N) static_cast<float*>(out)[row + n] = B ? acc[mi][nb][v] + bb[nb] : acc[mi][nb][v];
          }
        }
      }
    }
  };
  if (has_bias)
    plain(std::true_type{});
  else
    plain(std::false_type{});
}

// A thread's 128 accumulators as 32 float4 chunks (chunk 4 mi + nb is block
// (mi, nb)), chunk c of thread i at part[c * NTHR + i] of its piece: each
// chunk store is one coalesced 8 KiB.
__device__ __forceinline__ void store_partial(float4* __restrict__ part, const f32x4 (&acc)[8][4]) {
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      part[(mi * 4 + nb) * NTHR + threadIdx.x] = make_float4(acc[mi][nb][0], acc[mi][nb][1], acc[mi][nb][2], acc[mi][nb][3]);
}

template <bool GATED>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ gather,
    const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ B0,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ bias0,
    const uint16_t* __restrict__ bias1, void* __restrict__ out, uint16_t* __restrict__ resid, RopeOut ro, int N,
    int K, int NT, float4* __restrict__ part, int cus) {
  constexpr int COLS = GATED ? BNR / 2 : BNR;  // output columns per tile
  // Work unit -> tile (and K piece).  Units past the last one exit.
  const SplitPlan plan = split_plan(count_tiles(offsets, E, NT), cus, K / BK, part != nullptr);
  const int L = blockIdx.x;
  int tile = L, piece = -1;
  if (L >= plan.full) {
    const int u = L - plan.full;
    if (u >= plan.R * plan.S) return;
    tile = plan.full + u / plan.S;
    piece = u;
  }
  Tile t;
  if (!map_tile(offsets, E, NT, COLS, tile, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Copy sources.  Group 0: the activation rows (gathered through
  // sorted_token for the up projection; for the down projection the tile's
  // rows of h are contiguous, so the descriptor starts at the tile).  Group 1:
  // the tile's weight rows of W1 (waves 4, 5) or W3 (waves 6, 7) in the up
  // projection, of W2 in the down projection.  Every offset stays below 4 GiB:
  // a gathered row index is below T and the host requires T*d below 2^31
  // elements; every other descriptor starts at the tile's first row and
  // covers at most 256 rows of K elements.
  CopySrc cs;
  const uint16_t* base;
  if (wave < 4) {
    base = gather ? A : A + static_cast<int64_t>(t.m0) * K;
  } else {
    const uint16_t* Bm = (GATED && (wave & 3) >= 2) ? B1 : B0;
    base = Bm + (static_cast<int64_t>(t.e) * N + t.n0) * K;
  }
  cs.rsrc = wave_rsrc(base);
#pragma unroll
  for (int j = 0; j < COPIES; ++j) {
    const int r = (wave & 3) * 64 + j * 16 + (lane >> 2);
    const int chunk = (lane & 3) ^ ((r >> 2) & 3);
    int row;
    if (wave < 4) {
      const int rr = min(r, t.rows - 1);
      row = gather ? gather[t.m0 + rr] : rr;
    } else {
      row = min(GATED ? (r & 127) : r, N - 1 - t.n0);
    }
    cs.off[j] = (static_cast<uint32_t>(row) * K + chunk * 8) * 2;
  }

  // A piece covers slice pairs [p KP / S, (p + 1) KP / S) of the KP = KT / 2
  // pairs (at least 2 pairs: S <= KT / 4).
  int Kp = K;
  if (piece >= 0) {
    const int KP = K / (2 * BK);
    const int p = piece % plan.S;
    const int s0 = 2 * (p * KP / plan.S), s1 = 2 * ((p + 1) * KP / plan.S);
#pragma unroll
    for (int j = 0; j < COPIES; ++j) cs.off[j] += static_cast<uint32_t>(s0) * (BK * 2);
    Kp = (s1 - s0) * BK;
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mi][nb][v] = 0.f;

  // Every 32-row block holds at least one row once rows > BM - 32: the
  // branch-free path then does all MFMAs (at most one 16-row block of them
  // on clamped rows, whose results are not stored).
  if (t.rows > BM - 32)
    mainloop<GATED, true>(cs, Kp, t.rows, acc);
  else
    mainloop<GATED, false>(cs, Kp, t.rows, acc);

  if (piece >= 0)
    store_partial(part + static_cast<int64_t>(piece) * ACC_CHUNKS * NTHR, acc);
  else
    store_tile<GATED>(t, acc, bias0, bias1, out, resid, ro, N);
}

// Fix-up of the split tiles: workgroup 4 b + mi sums, for 32-row block mi of
// every wave, the S partial sums of split tile b in piece order and runs that
// block's epilogue (four workgroups per tile spread the partial-sum reads over
// more CUs).  Same thread layout as the GEMM kernel.
template <bool GATED>
__global__ __launch_bounds__(NTHR) void gemm_fixup_kernel(const int32_t* __restrict__ offsets, int E,
                                                          const uint16_t* __restrict__ bias0,
                                                          const uint16_t* __restrict__ bias1,
                                                          void* __restrict__ out, uint16_t* __restrict__ resid,
                                                          RopeOut ro, int N, int K, int NT,
                                                          const float4* __restrict__ part, int cus) {
  constexpr int COLS = GATED ? BNR / 2 : BNR;
  const SplitPlan plan = split_plan(count_tiles(offsets, E, NT), cus, K / BK, true);
  const int b = blockIdx.x >> 2, mb = blockIdx.x & 3;
  if (b >= plan.R) return;
  Tile t;
  if (!map_tile(offsets, E, NT, COLS, plan.full + b, t)) return;
  if (mb * 32 >= t.rows) return;  // no valid row in this block of either wave row
  f32x4 acc[8][4];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mi][nb][v] = 0.f;
  for (int p = 0; p < plan.S; ++p) {
    const float4* src = part + (static_cast<int64_t>(b) * plan.S + p) * ACC_CHUNKS * NTHR;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      if ((mi >> 1) != mb) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float4 v = src[(mi * 4 + nb) * NTHR + threadIdx.x];
        acc[mi][nb][0] += v.x;
        acc[mi][nb][1] += v.y;
        acc[mi][nb][2] += v.z;
        acc[mi][nb][3] += v.w;
      }
    }
  }
  store_tile<GATED>(t, acc, bias0, bias1, out, resid, ro, N, mb, mb + 1);
}

// Workgroups that run at once: one per CU (the LDS ring takes a CU's LDS),
// capped at the pieces the partial-sum buffer holds.
int concurrent_tiles() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = kGemmMaxPieces;
  return cus < kGemmMaxPieces ? cus : kGemmMaxPieces;
}

template <bool GATED>
hipError_t launch(const uint16_t* A, const int32_t* gather, const int32_t* offsets, const uint16_t* B0,
                  const uint16_t* B1, const uint16_t* bias0, const uint16_t* bias1, void* out, uint16_t* resid,
                  const RopeOut& ro, int64_t rows, int N, int K, int E, float* part, hipStream_t s) {
  constexpr int COLS = GATED ? BNR / 2 : BNR;
  const int NT = (N + COLS - 1) / COLS;
  const int cus = concurrent_tiles();
  // Upper bound on the row tiles: sum_e ceil(n_e / BM) <= ceil(rows / BM) + E;
  // splitting adds at most cus work units (R * S <= cus).
  const int64_t tiles = ((rows + BM - 1) / BM + E) * NT;
  // Only a kernel of a few rounds ends in one synchronised partial round: over
  // many rounds the tiles' durations differ, the rounds drift apart and the
  // end is ragged anyway (measured: no gain at 15 rounds, 13-26 % at 1-3).  So
  // with at least 4 rounds for certain (ceil(rows / BM) * NT tiles at least)
  // nothing is split and the fix-up is not launched.
  if (((rows + BM - 1) / BM) * NT >= 4 * static_cast<int64_t>(cus)) part = nullptr;
  // One expert owning every row (the attention projections) has exactly
  // ceil(rows / BM) * NT tiles: when they fill whole rounds nothing is split,
  // and the fix-up launch is skipped.  (Not splitting is correct for any
  // offsets; it only leaves a partial last round unsplit.)
  if (E == 1 && ((rows + BM - 1) / BM) * NT % cus == 0) part = nullptr;
  const int64_t units = part ? tiles + cus : tiles;
  float4* p4 = reinterpret_cast<float4*>(part);
  gemm_bf16_kernel<GATED><<<static_cast<unsigned>(units), NTHR, 0, s>>>(A, gather, offsets, E, B0, B1, bias0,
                                                                         bias1, out, resid, ro, N, K, NT, p4, cus);
  const hipError_t err = hipGetLastError();
  if (part == nullptr || err != hipSuccess) return err;
  // The split tiles number at most cus / 2 (S >= 2), four workgroups each.
  gemm_fixup_kernel<GATED><<<static_cast<unsigned>(cus / 2 * 4), NTHR, 0, s>>>(offsets, E, bias0, bias1, out,
                                                                               resid, ro, N, K, NT, p4, cus);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_up_bf16(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_token,
                               const uint16_t* w1, const uint16_t* w3, const uint16_t* b1,
                               const uint16_t* b3, uint16_t* h, int64_t T, int k, int d, int d_ff, int E,
                               float* part, hipStream_t stream) {
  return launch<true>(x, sorted_token, offsets, w1, w3, b1, b3, h, nullptr, RopeOut{}, T * k, d_ff, d, E, part,
                      stream);
}

hipError_t launch_gemm_down_bf16(const uint16_t* h, const int32_t* offsets, const uint16_t* w2,
                                 const uint16_t* b2, float* y_sorted, int64_t T, int k, int d, int d_ff,
                                 int E, float* part, hipStream_t stream) {
  return launch<false>(h, nullptr, offsets, w2, nullptr, b2, nullptr, y_sorted, nullptr, RopeOut{}, T * k, d, d_ff,
                       E, part, stream);
}

hipError_t launch_gemm_down_residual_bf16(const uint16_t* a, const int32_t* offsets, const uint16_t* w,
                                          const uint16_t* b, uint16_t* resid, int64_t rows, int N, int K, int E,
                                          float* part, hipStream_t stream) {
  return launch<false>(a, nullptr, offsets, w, nullptr, b, nullptr, nullptr, resid, RopeOut{}, rows, N, K, E, part,
                       stream);
}

hipError_t launch_gemm_qkv_rope_bf16(const uint16_t* a, const int32_t* offsets, const uint16_t* w,
                                     const float* cs, uint16_t* q, uint16_t* k, uint16_t* v, int64_t rows, int nq,
                                     int nkv, int K, float* part, hipStream_t stream) {
  const RopeOut ro{q, k, v, reinterpret_cast<const float2*>(cs), nq, nkv};
  return launch<false>(a, nullptr, offsets, w, nullptr, nullptr, nullptr, nullptr, nullptr, ro, rows, nq + 2 * nkv,
                       K, 1, part, stream);
}

}  // namespace moe
