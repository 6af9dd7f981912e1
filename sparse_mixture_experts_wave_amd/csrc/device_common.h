// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 (lo in the low half), round to nearest even, one
// instruction (v_cvt_pk_bf16_f32); equal to f32_to_bf16 on finite values.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// The low / high bf16 of a packed 32-bit word, widened.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// A raw buffer descriptor over [base, base + 4 GiB).  base must be the same in
// every lane of the wave; reading it through readfirstlane keeps the
// descriptor in scalar registers.  (Both halves are widened as unsigned: a
// sign-extended low half would corrupt the high half of the address.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* base) {
  const uint64_t bits = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bits)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bits >> 32)));
  // Raw buffer: stride 0, num_records = 4 GiB - 1 bytes, 32-bit data format word.
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), (short)0,
                                           static_cast<int>(0xFFFFFFFFu), 0x00020000);
}

// A 16-byte buffer load at byte offset voff + soff (soff wave-uniform) with the
// non-temporal cache policy: for data read once, such as streamed weights.
__device__ __forceinline__ u32x4 load16_buf_nt(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 2));
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// SiLU(z) = z / (1 + e^{-z}).  The fast form multiplies by the hardware
// reciprocal (v_rcp_f32, about 1 ulp) instead of dividing: an IEEE division
// is about ten vector instructions, and the up projection's epilogue forms
// one SiLU per output.  The result is rounded to bf16 afterwards.
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float silu_exact(float z) { return z / (1.0f + expf(-z)); }

// Which expert owns global M-tile `tile` when expert e contributes
// ceil(n_e / BM) tiles in expert order.  Returns -1 past the last tile.
// `first_row` receives the first sorted row of the tile, `rows` its row count.
template <int BM>
__device__ __forceinline__ int tile_to_expert(const int32_t* __restrict__ offsets, int E, int tile,
                                              int* first_row, int* rows) {
  int cum = 0;
  for (int e = 0; e < E; ++e) {
    const int lo = offsets[e];
    const int n = offsets[e + 1] - lo;
    const int t = (n + BM - 1) / BM;
    if (tile < cum + t) {
      const int local = tile - cum;
      *first_row = lo + local * BM;
      const int left = n - local * BM;
      *rows = left < BM ? left : BM;
      return e;
    }
    cum += t;
  }
  return -1;
}

}  // namespace moe
