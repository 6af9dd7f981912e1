// The attention sublayer around the MoE ("Mixtral" textbook page, section
// "Прямой проход в формулах": U = H + GQA(RMSNorm_1(H)), with
// Q_h = RoPE(X W_Q^h), K_c = RoPE(X W_K^c), V_c = X W_V^c,
// O_h = softmax(Q_h K_kappa(h)^T / sqrt(d_h) + M) V_kappa(h), kappa(h) = h / (H/G),
// M the causal mask, GQA(X) = [O_0; ...; O_{H-1}] W_O).
//
// Kernels here: a row RMSNorm, the RoPE rotation that also splits the fused
// Q|K|V projection into bf16 head-major tensors, the causal GQA flash
// attention, and the residual add after W_O.  The two projections run on the
// grouped MFMA GEMM of the experts (one "expert", no gather); on that path the
// GEMM's epilogues do the RoPE split (from the angle table the RMSNorm kernel
// writes) and the residual add themselves, and the RoPE and residual kernels
// here serve the streaming projections of a few tokens.
//
// RoPE reading: the page defers the rotation to another chapter; its
// HuggingFace loader permutes the rows of q_proj / k_proj per head, which
// turns HF's half-split rotation into the interleaved one.  So pair
// (2i, 2i+1) of a head vector at position p turns by p * theta^(-2i/d_h).
//
// Flash attention.  A 512-thread workgroup owns 256 queries of one head (32
// per wave, two waves per SIMD) and walks the key axis in 64-key tiles up to
// the diagonal.  Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16,
// so that a lane's accumulator column is one query: the running max, the
// exponentials and the running sum of a query stay in its lane and the lane 32
// apart (one cross-lane exchange per tile).  P^T then feeds O^T = V^T P^T
// straight from registers as the B operand: the k-index order of the MFMA is
// taken to be the order in which the S^T accumulator holds the keys, and V^T
// is read from LDS in that same order.  K is staged in LDS as [key][d_h] in
// 272-byte rows, V transposed, [d_h][key], in 144-byte rows with the keys of
// each 16-key group reordered so that every operand is one 16-byte read; the
// operand reads of both are free of bank conflicts.  The next tile's S MFMAs are
// interleaved with the current tile's softmax (see the kernel below).
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// RMSNorm of rows: u = x / sqrt(mean x^2 + eps) * gamma, rounded to bf16
// ---------------------------------------------------------------------------
constexpr int RN_T = 256;

// RoPE angle of pair i of a d_h-wide head at position pos, (cos, sin).  The
// angle is taken in fp64: positions reach 10^4 .. 10^5 and an fp32 angle would
// be off by up to ~1e-2 rad there.
__device__ __forceinline__ float2 rope_angle(int64_t pos, int i, int dh, double theta) {
  const double ang = static_cast<double>(pos) * pow(theta, -2.0 * i / dh);
  double sd, cd;
  sincos(ang, &sd, &cd);
  return make_float2(static_cast<float>(cd), static_cast<float>(sd));
}

// With cs set, workgroup t also writes the angles of position pos0 + t for
// the 64 pairs of a 128-wide head: cs[t][i], for the projection's epilogue.
// Workgroup 0 also writes row_range = [0, T] (one grid row per token), the
// offsets that let the expert GEMM run the projections as one expert owning
// every row.
__global__ __launch_bounds__(RN_T) void rmsnorm_rows_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ gamma, float eps,
                                                            uint16_t* __restrict__ u, int d,
                                                            int32_t* __restrict__ row_range,
                                                            float2* __restrict__ cs, double theta, int64_t pos0) {
  static_assert(RN_T >= 64, "one thread per angle");
  if (blockIdx.x == 0 && threadIdx.x < 2)
    row_range[threadIdx.x] = threadIdx.x == 0 ? 0 : static_cast<int32_t>(gridDim.x);
  if (cs && threadIdx.x < 64)
    cs[static_cast<int64_t>(blockIdx.x) * 64 + threadIdx.x] =
        rope_angle(pos0 + blockIdx.x, static_cast<int>(threadIdx.x), 128, theta);
  __shared__ float part[RN_T / kWave];
  const uint16_t* xr = x + static_cast<int64_t>(blockIdx.x) * d;
  uint16_t* ur = u + static_cast<int64_t>(blockIdx.x) * d;
  float ss = 0.f;
  for (int j = threadIdx.x * 8; j < d; j += RN_T * 8) {
    const u32x4 w = load16(xr + j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = lo_bf16(w[i]), b = hi_bf16(w[i]);
      ss += a * a + b * b;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < RN_T / kWave; ++w) tot += part[w];
  const float rinv = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
  for (int j = threadIdx.x * 8; j < d; j += RN_T * 8) {
    const u32x4 w = load16(xr + j);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_bf16x2(lo_bf16(w[i]) * rinv * gamma[j + 2 * i], hi_bf16(w[i]) * rinv * gamma[j + 2 * i + 1]);
    store16(ur + j, o);
  }
}

// ---------------------------------------------------------------------------
// RoPE + split: qkv fp32 [T][(H + 2G) d_h] -> q [T][H][d_h], k, v [T][G][d_h] bf16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rope_pack_kernel(const float* __restrict__ qkv, uint16_t* __restrict__ q,
                                                        uint16_t* __restrict__ k, uint16_t* __restrict__ v,
                                                        int64_t T, int H, int G, int dh, double theta,
                                                        int64_t pos0) {
  const int half = dh / 2;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= T * half) return;
  const int64_t t = idx / half;
  const int i = static_cast<int>(idx - t * half);
  const float2 a = rope_angle(pos0 + t, i, dh, theta);
  const float c = a.x, s = a.y;
  const float* row = qkv + t * static_cast<int64_t>(H + 2 * G) * dh + 2 * i;
  // Unrolled so that several heads' loads are in flight at once.
#pragma unroll 8
  for (int hh = 0; hh < H + G; ++hh) {
    const float2 x = *reinterpret_cast<const float2*>(row + static_cast<int64_t>(hh) * dh);
    const uint32_t r = pack_bf16x2(x.x * c - x.y * s, x.x * s + x.y * c);
    uint16_t* dst = hh < H ? q + (t * H + hh) * dh : k + (t * G + (hh - H)) * dh;
    *reinterpret_cast<uint32_t*>(dst + 2 * i) = r;
  }
#pragma unroll 8
  for (int gg = 0; gg < G; ++gg) {
    const float2 x = *reinterpret_cast<const float2*>(row + static_cast<int64_t>(H + G + gg) * dh);
    *reinterpret_cast<uint32_t*>(v + (t * G + gg) * dh + 2 * i) = pack_bf16x2(x.x, x.y);
  }
}

// ---------------------------------------------------------------------------
// residual: h += y (fp32), one rounding to bf16
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void residual_add_kernel(uint16_t* __restrict__ h, const float* __restrict__ y,
                                                           int64_t n8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const u32x4 w = load16(h + 8 * i);
  const float4 a = *reinterpret_cast<const float4*>(y + 8 * i);
  const float4 b = *reinterpret_cast<const float4*>(y + 8 * i + 4);
  u32x4 o;
  o[0] = pack_bf16x2(lo_bf16(w[0]) + a.x, hi_bf16(w[0]) + a.y);
  o[1] = pack_bf16x2(lo_bf16(w[1]) + a.z, hi_bf16(w[1]) + a.w);
  o[2] = pack_bf16x2(lo_bf16(w[2]) + b.x, hi_bf16(w[2]) + b.y);
  o[3] = pack_bf16x2(lo_bf16(w[3]) + b.z, hi_bf16(w[3]) + b.w);
  store16(h + 8 * i, o);
}

// ---------------------------------------------------------------------------
// causal GQA flash attention, d_h = 128
// ---------------------------------------------------------------------------
// A workgroup takes 256 queries of one head: eight waves (two per SIMD) of 32
// queries, walking 64-key tiles up to the diagonal.  Each wave computes
// S^T = K Q^T so that a lane's accumulator column is one query: the running
// max, the exponentials and the running sum stay in the lane (one exchange
// with the lane 32 apart per tile), and P^T feeds O^T = V^T P^T as the B
// operand straight from registers, the MFMA's k order taken to be the order in
// which the S^T accumulator holds the keys; V is staged transposed in LDS.
// The softmax is rescaled lazily: the reference max moves only when a tile's
// max exceeds it by more than 8 (log2 units).  The heads of one K/V group run
// on one XCD, the longest query tiles first.
//
// Software pipelining.  Per tile j a wave runs, in order:
//   A: S(j+1) for keys 0..31 of tile j+1 (8 MFMAs) beside tile j's row max;
//   (the lazy-rescale branch, rarely taken);
//   B: S(j+1) for keys 32..63 beside exp / sum / bf16 packing of tile j's
//      keys 0..31;
//   C: O(j) for keys 0..31 (8 MFMAs) beside the same for keys 32..63;
//   D: O(j) for keys 32..63 beside the stores of the next tiles into LDS.
// So the matrix core always has MFMAs that do not wait on the softmax.  K and
// V^T have two LDS buffers each: while tile j is consumed, K(j+2) goes into the
// buffer K(j) used and V(j+1) into the buffer V(j-1) used, so one barrier per
// tile suffices.
constexpr int FA_D = 128;                // head dimension
constexpr int FA_BKV = 64;               // keys per tile
constexpr int VT_STRIDE = FA_BKV + 8;    // 72 bf16 = 144 bytes per transposed V row

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }


// 2^x with the hardware instruction alone (v_exp_f32): results below 2^-126
// flush to zero instead of being rebuilt as denormals, which a softmax weight
// that small never needs (exp2f would spend about six instructions on it).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr bf16x2 kOnesBf16x2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

constexpr int FA_NW = 8;                   // waves per workgroup
constexpr int FA_QW = 32;                  // queries per wave
constexpr int FA_BQ = FA_QW * FA_NW;       // queries per workgroup
constexpr int FA_NT = 64 * FA_NW;
constexpr int FA_LD = FA_D + 8;            // padded K row: 272 bytes
constexpr int FA_KC = FA_BKV * FA_D / 8 / FA_NT;  // 16-byte K chunks per thread per tile (2)

// K rows padded to 272 bytes: the 16 rows one operand read touches start
// 4 banks apart (conflict-free), and every chunk of a lane's row is a constant
// offset from one address.
__device__ __forceinline__ int kpad(int row, int chunk) { return row * FA_LD + chunk * 8; }

// Column of key kk (0..63) in a transposed V row.  Within each 16-key group
// the keys are reordered so that the eight keys one lane feeds to an MFMA
// step (4 q + 0..3 and 8 + 4 q + 0..3 for lane half q) are adjacent: key
// 4 q + 8 h + i of the group goes to column 8 q + 4 h + i.  Rows of 144 bytes
// keep the 16-byte operand reads aligned and the 16 rows of one read in
// distinct banks.
__device__ __forceinline__ int vt_col(int kk) {
  const int r = kk & 15;
  return (kk & ~15) + 8 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

__global__ __launch_bounds__(FA_NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void flash_attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, int T, int H, int G, float scale_log2) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][FA_BKV * FA_LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][FA_D * VT_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[FA_NW][FA_QW * FA_LD];

  // Workgroups go to the 8 XCDs in turn by linear id, and gridDim.x = H: with
  // H a multiple of 8, XCD x gets heads x H/8 .. x H/8 + H/8 - 1, so the heads
  // that share a K/V group read it through one XCD's L2 (with the heads of a
  // group on different XCDs each L2 fetched K and V again: 2.8x the HBM reads).
  const int h = (H % 8 == 0) ? static_cast<int>(blockIdx.x % 8) * (H / 8) + static_cast<int>(blockIdx.x / 8)
                             : static_cast<int>(blockIdx.x);
  const int n_qt = (T + FA_BQ - 1) / FA_BQ;
  const int q0 = (n_qt - 1 - static_cast<int>(blockIdx.y)) * FA_BQ;  // longest rows first
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int qw = q0 + wave * FA_QW;        // first query of the wave
  const int my_q = qw + (lane & 31);       // the lane's query: its column of S^T and O^T
  const int64_t ld_q = static_cast<int64_t>(H) * FA_D;
  const int64_t ld_kv = static_cast<int64_t>(G) * FA_D;

  // B operand of S^T = K Q^T: lane holds query my_q (clamped to T - 1; its
  // output is not stored), dims 16 ks + 8 half .. +7.
  // Q goes through LDS: each wave loads its 32 rows four whole 256-byte rows
  // per instruction (row 4 i + lane / 16, chunk lane % 16), and reads the
  // operand layout back after the prologue's barrier.  Loaded straight into
  // the operand layout, every load instruction touched 32 rows.
  bf16x8 qf[8];
  u32x4 qraw[FA_QW / 4];
#pragma unroll
  for (int i = 0; i < FA_QW / 4; ++i)
    qraw[i] = load16(q + static_cast<int64_t>(min(qw + 4 * i + (lane >> 4), T - 1)) * ld_q + h * FA_D + 8 * (lane & 15));
  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int kv_end = min(T, q0 + FA_BQ);
  const int ntiles = (kv_end + FA_BKV - 1) / FA_BKV;
  // K/V staging through registers.  K: 16-byte chunks c = 2 tid, 2 tid + 1,
  // both of row tid / 8.  V: keys 2 kg, 2 kg + 1 (kg = tid % 32) x dims
  // 8 dg .. 8 dg + 7 (dg = tid / 32), stored transposed, the two keys side by
  // side at column vt_col(2 kg).  Keys past T are clamped to T - 1: they lie
  // above every query, so the mask removes them.  Row offsets are 32-bit
  // (24-bit multiplies): the launcher rejects T * G * d_h >= 2^31.
  static_assert(FA_KC == 2, "two K chunks per thread");
  const int kg = tid & 31, dg = tid >> 5;
  const uint32_t ld_kv32 = static_cast<uint32_t>(ld_kv);
  // Buffer loads through one descriptor per K and V head group, with 32-bit
  // byte offsets (below 2^32: the launcher rejects T * G * d_h >= 2^31): no
  // 64-bit address arithmetic per load (2 % of the kernel against global
  // loads).
  const __amdgpu_buffer_rsrc_t krs = wave_rsrc(k + g * FA_D);
  const __amdgpu_buffer_rsrc_t vrs = wave_rsrc(v + g * FA_D);
  const uint32_t kchunk = ((FA_KC * tid) & 15) * 16;  // bytes
  const uint32_t vchunk = 16 * dg;
  const uint32_t row_bytes = 2 * ld_kv32;
  const int vcol = vt_col(2 * kg);
  u32x4 kr[FA_KC], vr[2];
  auto load_k = [&](int kv0) {
    const uint32_t ro = __umul24(static_cast<uint32_t>(min(kv0 + (tid >> 3), T - 1)), row_bytes) + kchunk;
    kr[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, ro, 0, 0));
    kr[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, ro + 16, 0, 0));
  };
  auto load_v = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      vr[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     vrs, __umul24(static_cast<uint32_t>(min(kv0 + 2 * kg + i, T - 1)), row_bytes) + vchunk, 0, 0));
  };
  auto store_k_from = [&](int buf, const u32x4 (&src)[FA_KC]) {
#pragma unroll
    for (int i = 0; i < FA_KC; ++i) {
      const int c = tid * FA_KC + i;
      store16(&Ks[buf][kpad(c >> 4, c & 15)], src[i]);
    }
  };
  auto store_k = [&](int buf) { store_k_from(buf, kr); };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t e0 = (j & 1) ? hi16(vr[0][j >> 1]) : lo16(vr[0][j >> 1]);
      const uint32_t e1 = (j & 1) ? hi16(vr[1][j >> 1]) : lo16(vr[1][j >> 1]);
      *reinterpret_cast<uint32_t*>(&Vt[buf][(8 * dg + j) * VT_STRIDE + vcol]) = e0 | (e1 << 16);
    }
  };
  // S^T of keys 32 kb .. 32 kb + 31 of the tile in buffer buf: rows = keys
  // 32 kb + 8 (e / 4) + 4 half + e % 4, column = my_q.
  auto s_half = [&](f32x16 (&s)[2], int buf, int kb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
    bf16x8 a[8];  // all eight operand reads first, so the MFMAs do not wait on each
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) a[ks] = as_bf16x8(load16(&Ks[buf][kpad(kb * 32 + (lane & 31), 2 * ks + half)]));
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], qf[ks], s[kb], 0, 0, 0);
  };
  // p = 2^(s scale - m) for keys 32 kb .. + 31, their sum into lt, and the bf16
  // B operands of O^T += V^T P^T for the two 16-key steps of kb.
  auto softmax_half = [&](const f32x16 (&s)[2], int kb, float& lt, u32x4 (&pw)[2]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int e = 8 * hf + 2 * t;
        const float p0 = exp2_fast(fmaf(s[kb][e], scale_log2, -m));
        const float p1 = exp2_fast(fmaf(s[kb][e + 1], scale_log2, -m));
        // The row sum adds the bf16 weights the O MFMAs use: v_dot2 with
        // (1, 1), one instruction per pair.  (The packed word is copied to a
        // scalar first: a bit cast of an element of a vector variable reads
        // the wrong element with this compiler.)
        const uint32_t pp = cvt_pk_bf16(p0, p1);
        pw[hf][t] = pp;
        lt = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pp), kOnesBf16x2, lt, false);
      }
  };
  // O^T += V^T P^T over the two 16-key steps of keys 32 kb .. + 31.  Step hf
  // takes accumulator entries e = 8 hf .. +7, i.e. for lane half q the keys
  // 16 g + 4 q + 0..3 and 16 g + 8 + 4 q + 0..3 of 16-key group g = 2 kb + hf,
  // which V^T holds in that order at columns 16 g + 8 q .. + 7: one 16-byte
  // operand read each.
  auto o_half = [&](int buf, int kb, const u32x4 (&pw)[2]) {
    u32x4 aw[2][4];  // all operand reads first
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        aw[hf][db] = load16(&Vt[buf][(db * 32 + (lane & 31)) * VT_STRIDE + 16 * (2 * kb + hf) + 8 * half]);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(aw[hf][db]), as_bf16x8(pw[hf]), oacc[db], 0, 0, 0);
  };

  // One tile: sc holds S^T of tile j, sn receives S^T of tile j + 1.
  auto tile = [&](int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    const int kv0 = j * FA_BKV;
    const int buf = j & 1;
    // Loads and stores run on every tile, past the last one too: their key
    // rows are clamped to T - 1, and such a store lands in a buffer that
    // nothing reads again but the S of a tile past the end.  Guarded loads
    // made the compiler wait for each tile's K loads before it issued the V
    // loads.
    load_k(kv0 + 2 * FA_BKV);
    load_v(kv0 + FA_BKV);
    if (kv0 <= qw + FA_QW - 1) {  // some key of tile j is visible to some query of the wave
      if (kv0 + FA_BKV - 1 > qw) {  // causal mask on the diagonal tiles only
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (kv0 + kb * 32 + 8 * (e >> 2) + 4 * half + (e & 3) > my_q) sc[kb][e] = -INFINITY;
      }
      // A: S(j+1), keys 0..31, beside the row max of tile j.
      s_half(sn, buf ^ 1, 0);
      float x = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) x = fmaxf(x, sc[kb][e]);
      const float mt = fmaxf(x, __shfl_xor(x, 32)) * scale_log2;
      // Lazy rescaling: the reference max m only moves when the tile's max
      // exceeds it by more than 8, so every p = 2^(s - m) stays <= 2^8 and the
      // rescale of O and l is skipped on most tiles.  O / l does not depend on
      // m.  m is finite after the first tile: key 0 is visible to every query.
      if (__ballot(mt > m + 8.f)) {
        const float m_new = mt > m + 8.f ? mt : m;
        const float alpha = exp2_fast(m - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        m = m_new;
      }
      float lt = 0.f;
      u32x4 pw0[2], pw1[2];
      // B: S(j+1), keys 32..63, beside the softmax of tile j's keys 0..31.
      s_half(sn, buf ^ 1, 1);
      softmax_half(sc, 0, lt, pw0);
      // C: O(j), keys 0..31, beside the softmax of keys 32..63.
      o_half(buf, 0, pw0);
      softmax_half(sc, 1, lt, pw1);
      // D: O(j), keys 32..63.
      o_half(buf, 1, pw1);
      l += lt + __shfl_xor(lt, 32);
    }
    store_k(buf);
    store_v(buf ^ 1);
    __syncthreads();
  };

  // Prologue: K(0), V(0) and K(1) into LDS, then S^T of tile 0.  The three
  // loads go out together (K(1) into spare registers; rows clamped like every
  // tile's), so the workgroup waits for one memory round trip, not two.
  u32x4 k1[FA_KC];
  load_k(FA_BKV);
  k1[0] = kr[0];
  k1[1] = kr[1];
  load_k(0);
  load_v(0);
#pragma unroll
  for (int i = 0; i < FA_QW / 4; ++i) store16(&Qs[wave][(4 * i + (lane >> 4)) * FA_LD + 8 * (lane & 15)], qraw[i]);
  store_k(0);
  store_v(0);
  store_k_from(1, k1);
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(load16(&Qs[wave][(lane & 31) * FA_LD + 16 * ks + 8 * half]));
  f32x16 sA[2], sB[2];
  s_half(sA, 0, 0);
  s_half(sA, 0, 1);
  for (int j = 0; j < ntiles; j += 2) {
    tile(j, sA, sB);
    if (j + 1 < ntiles) tile(j + 1, sB, sA);
  }

  // O^T accumulator: lane holds query my_q, dims 32 db + 8 (e / 4) + 4 half + e % 4,
  // so each group of four e is four adjacent dims.  The wave's 32 x 128 block
  // of O goes through LDS (the K / V buffers are free after the last tile's
  // barrier: waves 0-3 use Ks, 4-7 Vt, 32 rows of 272 bytes each) and out as
  // whole 256-byte rows, four per store instruction.  Stored straight from the
  // accumulator layout, every store instruction touched 32 rows and the
  // workgroup's stores took several microseconds to drain.
  {
    const float inv = 1.0f / l;
    static_assert(FA_NW / 2 * FA_QW * FA_LD * 2 <= static_cast<int>(sizeof(Ks)), "O staging exceeds Ks");
    static_assert(FA_NW / 2 * FA_QW * FA_LD * 2 <= static_cast<int>(sizeof(Vt)), "O staging exceeds Vt");
    uint16_t* stage = (wave < FA_NW / 2 ? &Ks[0][0] : &Vt[0][0]) + (wave % (FA_NW / 2)) * FA_QW * FA_LD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int e = 4 * g4;
        uint2 w;
        w.x = cvt_pk_bf16(oacc[db][e] * inv, oacc[db][e + 1] * inv);
        w.y = cvt_pk_bf16(oacc[db][e + 2] * inv, oacc[db][e + 3] * inv);
        *reinterpret_cast<uint2*>(&stage[(lane & 31) * FA_LD + db * 32 + 8 * g4 + 4 * half]) = w;
      }
    __syncthreads();
    // Store instruction i: rows 4 i + lane / 16 of the wave, 16-byte chunk lane % 16.
#pragma unroll
    for (int i = 0; i < FA_QW / 4; ++i) {
      const int r = 4 * i + (lane >> 4);
      const int c = lane & 15;
      const u32x4 v = load16(&stage[r * FA_LD + 8 * c]);
      if (qw + r < T) store16(o + static_cast<int64_t>(qw + r) * ld_q + h * FA_D + 8 * c, v);
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm_rows(const uint16_t* x, const float* gamma, float eps, uint16_t* u, int64_t T, int d,
                               int32_t* row_range, hipStream_t stream, float* cs, double theta, int64_t pos0) {
  rmsnorm_rows_kernel<<<static_cast<unsigned>(T), RN_T, 0, stream>>>(x, gamma, eps, u, d, row_range,
                                                                     reinterpret_cast<float2*>(cs), theta, pos0);
  return hipGetLastError();
}

hipError_t launch_rope_pack(const float* qkv, uint16_t* q, uint16_t* k, uint16_t* v, int64_t T, int H, int G,
                            int dh, double theta, int64_t pos0, hipStream_t stream) {
  const int64_t n = T * (dh / 2);
  rope_pack_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(qkv, q, k, v, T, H, G, dh, theta,
                                                                               pos0);
  return hipGetLastError();
}

hipError_t launch_residual_add(uint16_t* h, const float* y, int64_t n, hipStream_t stream) {
  const int64_t n8 = n / 8;
  residual_add_kernel<<<static_cast<unsigned>((n8 + 255) / 256), 256, 0, stream>>>(h, y, n8);
  return hipGetLastError();
}

bool flash_attn_supported(int dh) { return dh == FA_D; }

hipError_t launch_flash_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, int64_t T,
                             int H, int G, int dh, hipStream_t stream) {
  if (T * G * static_cast<int64_t>(dh) >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  const float scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(dh)));
  const dim3 grid(static_cast<unsigned>(H), static_cast<unsigned>((T + FA_BQ - 1) / FA_BQ));
  flash_attn_fwd_kernel<<<grid, FA_NT, 0, stream>>>(q, k, v, o, static_cast<int>(T), H, G, scale_log2);
  return hipGetLastError();
}

}  // namespace moe
