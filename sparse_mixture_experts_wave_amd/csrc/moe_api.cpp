// C ABI of the MoE layer: argument validation, workspace carving and the
// launch sequence route -> dispatch -> experts -> combine (and, for the
// attention sublayer, rmsnorm -> qkv -> rope -> attention -> output -> residual).  Host code,
// plus one static device array (the scratch buffer of moe_forward_noalloc);
// every launch is asynchronous on the caller's stream and nothing here
// synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.h"
#include "moe.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

moe_status hip_status(hipError_t err, const char* what) {
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int32_t dt) { return dt == MOE_BF16 ? 2 : 4; }

// Shape rules shared by every entry point.
moe_status check_shape(const moe_shape* s) {
  if (s == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld < 0", static_cast<long long>(s->T));
  if (s->d <= 0 || s->d % 64 != 0 || s->d > 32768)
    return fail(MOE_ERR_INVALID_ARG, "d = %d must be a positive multiple of 64, at most 32768", s->d);
  if (s->d_ff <= 0 || s->d_ff % 64 != 0 || s->d_ff > 65536)
    return fail(MOE_ERR_INVALID_ARG, "d_ff = %d must be a positive multiple of 64, at most 65536", s->d_ff);
  if (s->E < 2 || s->E > 64) return fail(MOE_ERR_INVALID_ARG, "E = %d outside 2..64", s->E);
  if (s->k < 1 || s->k > s->E)
    return fail(MOE_ERR_INVALID_ARG, "top-k = %d outside 1..E (E = %d)", s->k, s->E);
  if (s->act != MOE_F32 && s->act != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "act dtype %d unknown", s->act);
  if (s->wt != MOE_F32 && s->wt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "wt dtype %d unknown", s->wt);
  if (s->k > moe::kRouterMaxK)
    return fail(MOE_ERR_UNSUPPORTED, "top-k = %d: at most %d is implemented", s->k, moe::kRouterMaxK);
  if ((s->E & (s->E - 1)) != 0) return fail(MOE_ERR_UNSUPPORTED, "E = %d is not a power of two", s->E);
  if (s->act != s->wt)
    return fail(MOE_ERR_UNSUPPORTED, "dtype pair (act %d, wt %d): only (f32, f32) and (bf16, bf16)", s->act, s->wt);
  // Row indices are int32 on the device.
  if (s->T > (int64_t{1} << 30) / s->k)
    return fail(MOE_ERR_INVALID_ARG, "T = %lld too large", static_cast<long long>(s->T));
  // The prefill GEMM addresses gathered activation rows with 32-bit byte offsets.
  if (s->T * s->d >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T * d = %lld: at most 2^31 - 1 activation elements per call",
                static_cast<long long>(s->T * s->d));
  return MOE_OK;
}

moe_status need(const void* p, const char* name) {
  if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

moe_status optional(const void* p, const char* name) {
  if (p != nullptr && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define MOE_TRY(expr)                 \
  do {                                \
    const moe_status st_ = (expr);    \
    if (st_ != MOE_OK) return st_;    \
  } while (0)

constexpr size_t kAlign = 256;
size_t up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Workspace layout of moe_forward / moe_block_forward.
struct Layout {
  size_t topk_idx, topk_w, offsets, sorted_token, inv_pos, h, y_sorted, u, part, total;
};

// Partial-sum buffer of the bf16 grouped GEMM (0 bytes on the streaming path).
size_t part_bytes(const moe_shape* s) {
  return s->wt == MOE_BF16 ? moe::gemm_partial_bytes(s->T, s->d, s->d_ff) : 0;
}

Layout layout(const moe_shape* s, bool block, bool with_part = true) {
  const size_t rows = static_cast<size_t>(s->T) * s->k;
  Layout L{};
  size_t at = 0;
  L.topk_idx = at; at += up(rows * 4);
  L.topk_w = at; at += up(rows * 4);
  L.offsets = at; at += up((s->E + 1) * 4);
  L.sorted_token = at; at += up(rows * 4);
  L.inv_pos = at; at += up(rows * 4);
  L.h = at; at += up(rows * s->d_ff * esize(s->wt));
  L.y_sorted = at; at += up(rows * s->d * 4);
  L.u = at; if (block) at += up(static_cast<size_t>(s->T) * s->d * esize(s->act));
  L.part = at; if (with_part) at += up(part_bytes(s));
  L.total = at;
  return L;
}

// moe_expert_ffn's workspace: h, then the partial-sum buffer.
size_t ffn_h_bytes(const moe_shape* s) { return up(static_cast<size_t>(s->T) * s->k * s->d_ff * esize(s->wt)); }
size_t ffn_ws(const moe_shape* s) { return ffn_h_bytes(s) + up(part_bytes(s)); }

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

hipStream_t hs(void* stream) { return static_cast<hipStream_t>(stream); }

moe_status run_route(const moe_shape* s, const void* x, const float* w_gate, const float* bias,
                     float* logits, int32_t* idx, float* w, const float* gamma, float eps,
                     void* u_out, void* stream) {
  return hip_status(moe::launch_route(x, s->act == MOE_BF16, w_gate, bias, logits, idx, w, s->T, s->d,
                                      s->E, s->k, gamma, eps, u_out, hs(stream)),
                    "router launch");
}

// Optional per-thread timing points (moe_set_timing_events).
thread_local hipEvent_t g_events[MOE_TIMING_POINTS];
thread_local bool g_timing = false;

moe_status mark(int point, void* stream) {
  if (!g_timing) return MOE_OK;
  return hip_status(hipEventRecord(g_events[point], hs(stream)), "timing event record");
}

// Optional expert biases: every pointer may be NULL, and so may the struct.
moe_status check_bias(const moe_expert_bias* eb) {
  if (eb == nullptr) return MOE_OK;
  MOE_TRY(optional(eb->b1, "expert_bias->b1"));
  MOE_TRY(optional(eb->b3, "expert_bias->b3"));
  return optional(eb->b2, "expert_bias->b2");
}

// Dispatch folded into the up projection: the router's choices in, the
// permutation (offsets, sorted_token, inv_pos) written by that kernel.
struct FusedDispatchArgs {
  const int32_t* topk_idx;
  int32_t* inv_pos;
};

moe_status run_ffn(const moe_shape* s, const void* x, const int32_t* off, const int32_t* st,
                   const void* w1, const void* w3, const void* w2, const moe_expert_bias* eb, float* y_sorted,
                   void* h, float* part, void* stream, bool timed, const FusedDispatchArgs* fused = nullptr) {
  const void* b1 = eb ? eb->b1 : nullptr;
  const void* b3 = eb ? eb->b3 : nullptr;
  const void* b2 = eb ? eb->b2 : nullptr;
  hipError_t err;
  if (fused != nullptr) {
    err = moe::launch_stream_up_dispatch_bf16(static_cast<const uint16_t*>(x), fused->topk_idx, s->k,
                                              const_cast<int32_t*>(off), const_cast<int32_t*>(st), fused->inv_pos,
                                              static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3),
                                              static_cast<const uint16_t*>(b1), static_cast<const uint16_t*>(b3),
                                              static_cast<uint16_t*>(h), s->T, s->d, s->d_ff, s->E, hs(stream));
  } else if (s->wt == MOE_BF16) {
    err = moe::launch_expert_up_bf16(static_cast<const uint16_t*>(x), off, st, static_cast<const uint16_t*>(w1),
                                     static_cast<const uint16_t*>(w3), static_cast<const uint16_t*>(b1),
                                     static_cast<const uint16_t*>(b3), static_cast<uint16_t*>(h), s->T, s->k,
                                     s->d, s->d_ff, s->E, part, hs(stream));
  } else {
    err = moe::launch_expert_up_f32(static_cast<const float*>(x), off, st, static_cast<const float*>(w1),
                                    static_cast<const float*>(w3), static_cast<const float*>(b1),
                                    static_cast<const float*>(b3), static_cast<float*>(h), s->T, s->k, s->d,
                                    s->d_ff, s->E, hs(stream));
  }
  MOE_TRY(hip_status(err, "expert up launch"));
  if (timed) MOE_TRY(mark(3, stream));
  if (s->wt == MOE_BF16) {
    err = moe::launch_expert_down_bf16(static_cast<const uint16_t*>(h), off, static_cast<const uint16_t*>(w2),
                                       static_cast<const uint16_t*>(b2), y_sorted, s->T, s->k, s->d, s->d_ff,
                                       s->E, part, hs(stream));
  } else {
    err = moe::launch_expert_down_f32(static_cast<const float*>(h), off, static_cast<const float*>(w2),
                                      static_cast<const float*>(b2), y_sorted, s->T, s->k, s->d, s->d_ff, s->E,
                                      hs(stream));
  }
  return hip_status(err, "expert down launch");
}

moe_status forward_impl(const moe_shape* s, const void* x, const float* w_gate, const float* bias,
                        const void* w1, const void* w3, const void* w2, const moe_expert_bias* eb, void* y,
                        const void* residual, const float* gamma, float eps, void* ws, size_t ws_bytes,
                        void* stream, bool with_part = true) {
  const bool block = gamma != nullptr;
  const Layout L = layout(s, block, with_part);
  if (ws_bytes < L.total)
    return fail(MOE_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", ws_bytes, L.total);
  int32_t* idx = at<int32_t>(ws, L.topk_idx);
  float* w = at<float>(ws, L.topk_w);
  int32_t* off = at<int32_t>(ws, L.offsets);
  int32_t* st = at<int32_t>(ws, L.sorted_token);
  int32_t* inv = at<int32_t>(ws, L.inv_pos);
  void* h = at<void>(ws, L.h);
  float* ys = at<float>(ws, L.y_sorted);
  const void* xin = x;
  void* u = nullptr;
  if (block) {
    u = at<void>(ws, L.u);
    xin = u;
  }
  // Decode-size bf16 layers sort the router's choices inside the streaming up
  // projection instead of in a dispatch launch of their own.
  const bool fuse = s->wt == MOE_BF16 && moe::stream_dispatch_supported(s->T, s->k, s->d, s->d_ff, s->E);
  const FusedDispatchArgs fused{idx, inv};
  MOE_TRY(mark(0, stream));
  MOE_TRY(run_route(s, x, w_gate, bias, nullptr, idx, w, gamma, eps, u, stream));
  MOE_TRY(mark(1, stream));
  if (!fuse)
    MOE_TRY(hip_status(moe::launch_dispatch(idx, s->T, s->k, s->E, off, st, inv, hs(stream)), "dispatch launch"));
  MOE_TRY(mark(2, stream));
  float* part = (with_part && part_bytes(s)) ? at<float>(ws, L.part) : nullptr;
  MOE_TRY(run_ffn(s, xin, off, st, w1, w3, w2, eb, ys, h, part, stream, true, fuse ? &fused : nullptr));
  MOE_TRY(mark(4, stream));
  MOE_TRY(hip_status(moe::launch_combine(ys, inv, w, residual, y, s->act == MOE_BF16, s->T, s->k, s->d, hs(stream)),
                     "combine launch"));
  return mark(5, stream);
}

// ---------------------------------------------------------------------------
// the layer without a caller workspace (moe_forward_noalloc)
// ---------------------------------------------------------------------------
// The intermediates of one moe_forward_noalloc call (routing, permutation, h,
// y_sorted; no GEMM partial sums) live in this array.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// `scratch` is only a host-side stand-in for the symbol: kernels get the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
moe_status scratch_address(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(err));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// attention sublayer
// ---------------------------------------------------------------------------
moe_status check_attn_shape(const moe_attn_shape* s) {
  if (s == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld < 0", static_cast<long long>(s->T));
  if (s->d <= 0 || s->d % 64 != 0 || s->d > 32768)
    return fail(MOE_ERR_INVALID_ARG, "d = %d must be a positive multiple of 64, at most 32768", s->d);
  if (s->H < 1 || s->G < 1 || s->H % s->G != 0 || s->H > 1024)
    return fail(MOE_ERR_INVALID_ARG, "H = %d, G = %d: need 1 <= G, H %% G == 0, H <= 1024", s->H, s->G);
  if (s->d_h <= 0 || s->d_h % 2 != 0) return fail(MOE_ERR_INVALID_ARG, "d_h = %d must be positive and even", s->d_h);
  if (s->act != MOE_F32 && s->act != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "act dtype %d unknown", s->act);
  if (!moe::flash_attn_supported(s->d_h)) return fail(MOE_ERR_UNSUPPORTED, "d_h = %d: only 128 is implemented", s->d_h);
  if (s->act != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "attention is implemented for bf16 only");
  const int64_t widest = std::max<int64_t>(s->d, static_cast<int64_t>(s->H + 2 * s->G) * s->d_h);
  if (s->T * widest >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T * %lld = %lld: at most 2^31 - 1 elements per activation tensor",
                static_cast<long long>(widest), static_cast<long long>(s->T * widest));
  return MOE_OK;
}

struct AttnLayout {
  size_t offsets, xn, qkv, cs, q, k, v, o, oproj, part, total;
};

AttnLayout attn_layout(const moe_attn_shape* s) {
  const size_t T = static_cast<size_t>(s->T);
  const size_t nq = static_cast<size_t>(s->H) * s->d_h, nkv = static_cast<size_t>(s->G) * s->d_h;
  AttnLayout L{};
  size_t at = 0;
  L.offsets = at; at += up(2 * 4);
  L.xn = at; at += up(T * s->d * 2);
  // The fp32 Q|K|V projection before RoPE: only the streaming path of a few
  // tokens writes it.  The GEMM path rotates in its epilogue, reading the
  // (cos, sin) table [T][64] that the RMSNorm kernel writes.
  const bool qkv_stream = moe::stream_supported(s->T, static_cast<int>(nq + 2 * nkv), s->d);
  L.qkv = at;
  if (qkv_stream) at += up(T * (nq + 2 * nkv) * 4);
  L.cs = at;
  if (!qkv_stream) at += up(T * 64 * 8);
  L.q = at; at += up(T * nq * 2);
  L.k = at; at += up(T * nkv * 2);
  L.v = at; at += up(T * nkv * 2);
  L.o = at; at += up(T * nq * 2);
  // The fp32 output projection before the residual add: only the streaming
  // path of a few tokens writes it (the GEMM adds into h in its epilogue).
  L.oproj = at;
  if (moe::stream_supported(s->T, s->d, static_cast<int>(nq))) at += up(T * s->d * 4);
  // The projections' GEMM partial sums (one buffer, used by one projection at a time).
  const size_t pb = std::max(moe::gemm_partial_bytes(s->T, static_cast<int>(nq + 2 * nkv), s->d),
                             moe::gemm_partial_bytes(s->T, s->d, static_cast<int>(nq)));
  L.part = at; at += up(pb);
  L.total = at;
  return L;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return layout(shape, true).total;
}

size_t moe_expert_ffn_workspace_size(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return ffn_ws(shape);
}

moe_status moe_route(const moe_shape* shape, const void* x, const float* w_gate, const float* bias,
                     float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  MOE_TRY(check_shape(shape));
  if (shape->T == 0) return ok();
  MOE_TRY(need(x, "x"));
  MOE_TRY(need(w_gate, "w_gate"));
  MOE_TRY(optional(bias, "bias"));
  MOE_TRY(optional(logits, "logits"));
  MOE_TRY(need(topk_idx, "topk_idx"));
  MOE_TRY(need(topk_w, "topk_w"));
  return run_route(shape, x, w_gate, bias, logits, topk_idx, topk_w, nullptr, 0.f, nullptr, stream);
}

moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, int32_t* expert_offsets,
                        int32_t* sorted_token, int32_t* inv_pos, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  MOE_TRY(check_shape(shape));
  MOE_TRY(need(expert_offsets, "expert_offsets"));
  // With T == 0 the offsets are still defined (all zero), so the kernel runs;
  // it touches no other buffer then.
  if (shape->T > 0) {
    MOE_TRY(need(topk_idx, "topk_idx"));
    MOE_TRY(need(sorted_token, "sorted_token"));
    MOE_TRY(need(inv_pos, "inv_pos"));
  }
  return hip_status(moe::launch_dispatch(topk_idx, shape->T, shape->k, shape->E, expert_offsets, sorted_token,
                                         inv_pos, hs(stream)),
                    "dispatch launch");
}

moe_status moe_expert_ffn(const moe_shape* shape, const void* x, const int32_t* expert_offsets,
                          const int32_t* sorted_token, const void* w1, const void* w3, const void* w2,
                          const moe_expert_bias* expert_bias, float* y_sorted, void* ws, size_t ws_bytes,
                          void* stream) {
  MOE_TRY(check_shape(shape));
  if (shape->T == 0) return ok();
  MOE_TRY(need(x, "x"));
  MOE_TRY(need(expert_offsets, "expert_offsets"));
  MOE_TRY(need(sorted_token, "sorted_token"));
  MOE_TRY(need(w1, "w1"));
  MOE_TRY(need(w3, "w3"));
  MOE_TRY(need(w2, "w2"));
  MOE_TRY(check_bias(expert_bias));
  MOE_TRY(need(y_sorted, "y_sorted"));
  MOE_TRY(need(ws, "ws"));
  if (ws_bytes < ffn_ws(shape))
    return fail(MOE_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", ws_bytes, ffn_ws(shape));
  float* part = part_bytes(shape) ? at<float>(ws, ffn_h_bytes(shape)) : nullptr;
  return run_ffn(shape, x, expert_offsets, sorted_token, w1, w3, w2, expert_bias, y_sorted, ws, part, stream,
                 false);
}

moe_status moe_combine(const moe_shape* shape, const float* y_sorted, const int32_t* inv_pos,
                       const float* topk_w, const void* residual, void* y, void* stream) {
  MOE_TRY(check_shape(shape));
  if (shape->T == 0) return ok();
  MOE_TRY(need(y_sorted, "y_sorted"));
  MOE_TRY(need(inv_pos, "inv_pos"));
  MOE_TRY(need(topk_w, "topk_w"));
  MOE_TRY(optional(residual, "residual"));
  MOE_TRY(need(y, "y"));
  return hip_status(moe::launch_combine(y_sorted, inv_pos, topk_w, residual, y, shape->act == MOE_BF16, shape->T,
                                        shape->k, shape->d, hs(stream)),
                    "combine launch");
}

moe_status moe_forward(const moe_shape* shape, const void* x, const float* w_gate, const float* bias,
                       const void* w1, const void* w3, const void* w2, const moe_expert_bias* expert_bias,
                       void* y, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_shape(shape));
  if (shape->T == 0) return ok();
  MOE_TRY(need(x, "x"));
  MOE_TRY(need(w_gate, "w_gate"));
  MOE_TRY(optional(bias, "bias"));
  MOE_TRY(need(w1, "w1"));
  MOE_TRY(need(w3, "w3"));
  MOE_TRY(need(w2, "w2"));
  MOE_TRY(check_bias(expert_bias));
  MOE_TRY(need(y, "y"));
  if (x == y) return fail(MOE_ERR_INVALID_ARG, "y must not alias x");
  MOE_TRY(need(ws, "ws"));
  return forward_impl(shape, x, w_gate, bias, w1, w3, w2, expert_bias, y, nullptr, nullptr, 0.f, ws, ws_bytes,
                      stream);
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_gate, const float* bias,
                               const void* w1, const void* w3, const void* w2, const moe_expert_bias* expert_bias,
                               void* y, void* stream) {
  MOE_TRY(check_shape(shape));
  if (shape->T == 0) return ok();
  MOE_TRY(need(x, "x"));
  MOE_TRY(need(w_gate, "w_gate"));
  MOE_TRY(optional(bias, "bias"));
  MOE_TRY(need(w1, "w1"));
  MOE_TRY(need(w3, "w3"));
  MOE_TRY(need(w2, "w2"));
  MOE_TRY(check_bias(expert_bias));
  MOE_TRY(need(y, "y"));
  if (x == y) return fail(MOE_ERR_INVALID_ARG, "y must not alias x");
  const size_t need_bytes = layout(shape, false, false).total;
  if (need_bytes > kNoAllocScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED,
                "T = %lld needs %zu bytes of intermediates; the static scratch buffer holds %zu (use moe_forward "
                "with a workspace)",
                static_cast<long long>(shape->T), need_bytes, kNoAllocScratchBytes);
  void* ws = nullptr;
  MOE_TRY(scratch_address(&ws));
  return forward_impl(shape, x, w_gate, bias, w1, w3, w2, expert_bias, y, nullptr, nullptr, 0.f, ws,
                      kNoAllocScratchBytes, stream, false);
}

moe_status moe_block_forward(const moe_shape* shape, void* h_inout, const float* gamma, float eps,
                             const float* w_gate, const float* bias, const void* w1, const void* w3,
                             const void* w2, const moe_expert_bias* expert_bias, void* ws, size_t ws_bytes,
                             void* stream) {
  MOE_TRY(check_shape(shape));
  if (!(eps > 0.f)) return fail(MOE_ERR_INVALID_ARG, "eps = %g must be > 0", static_cast<double>(eps));
  if (shape->T == 0) return ok();
  MOE_TRY(need(h_inout, "h_inout"));
  MOE_TRY(need(gamma, "gamma"));
  MOE_TRY(need(w_gate, "w_gate"));
  MOE_TRY(optional(bias, "bias"));
  MOE_TRY(need(w1, "w1"));
  MOE_TRY(need(w3, "w3"));
  MOE_TRY(need(w2, "w2"));
  MOE_TRY(check_bias(expert_bias));
  MOE_TRY(need(ws, "ws"));
  return forward_impl(shape, h_inout, w_gate, bias, w1, w3, w2, expert_bias, h_inout, h_inout, gamma, eps, ws,
                      ws_bytes, stream);
}

moe_status moe_aux_loss(const moe_shape* shape, const float* logits, int32_t num_layers,
                        const uint8_t* token_mask, float alpha, float* loss, float* stats, void* stream) {
  if (shape == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (shape->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld < 0", static_cast<long long>(shape->T));
  if (shape->E < 2 || shape->E > 64) return fail(MOE_ERR_INVALID_ARG, "E = %d outside 2..64", shape->E);
  if (shape->k < 1 || shape->k > shape->E)
    return fail(MOE_ERR_INVALID_ARG, "top-k = %d outside 1..E (E = %d)", shape->k, shape->E);
  if ((shape->E & (shape->E - 1)) != 0) return fail(MOE_ERR_UNSUPPORTED, "E = %d is not a power of two", shape->E);
  if (shape->k > moe::aux_loss_max_k())
    return fail(MOE_ERR_UNSUPPORTED, "top-k = %d above %d", shape->k, moe::aux_loss_max_k());
  if (num_layers < 1) return fail(MOE_ERR_INVALID_ARG, "num_layers = %d < 1", num_layers);
  if (!(alpha >= 0.f)) return fail(MOE_ERR_INVALID_ARG, "alpha = %g must be >= 0", static_cast<double>(alpha));
  MOE_TRY(need(loss, "loss"));
  MOE_TRY(optional(stats, "stats"));
  if (shape->T > 0) {
    MOE_TRY(need(logits, "logits"));
    if (token_mask != nullptr && (reinterpret_cast<uintptr_t>(token_mask) & 15u) != 0)
      return fail(MOE_ERR_INVALID_ARG, "token_mask is not 16-byte aligned");
  }
  return hip_status(moe::launch_aux_loss(logits, num_layers, shape->T, shape->E, shape->k, token_mask, alpha, loss,
                                         stats, hs(stream)),
                    "aux loss launch");
}

size_t moe_attention_workspace_size(const moe_attn_shape* shape) {
  if (check_attn_shape(shape) != MOE_OK) return 0;
  return attn_layout(shape).total;
}

moe_status moe_gqa_attention(const moe_attn_shape* shape, const void* q, const void* k, const void* v, void* o,
                             void* stream) {
  MOE_TRY(check_attn_shape(shape));
  if (shape->T == 0) return ok();
  MOE_TRY(need(q, "q"));
  MOE_TRY(need(k, "k"));
  MOE_TRY(need(v, "v"));
  MOE_TRY(need(o, "o"));
  return hip_status(moe::launch_flash_attn(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), shape->T,
                                           shape->H, shape->G, shape->d_h, hs(stream)),
                    "attention launch");
}

moe_status moe_attention_block_forward(const moe_attn_shape* shape, void* h_inout, const float* gamma, float eps,
                                       const void* wqkv, const void* wo, float rope_theta, int64_t pos0, void* ws,
                                       size_t ws_bytes, void* stream) {
  MOE_TRY(check_attn_shape(shape));
  if (!(eps > 0.f)) return fail(MOE_ERR_INVALID_ARG, "eps = %g must be > 0", static_cast<double>(eps));
  if (!(rope_theta > 0.f))
    return fail(MOE_ERR_INVALID_ARG, "rope_theta = %g must be > 0", static_cast<double>(rope_theta));
  if (pos0 < 0 || pos0 > (int64_t{1} << 40))
    return fail(MOE_ERR_INVALID_ARG, "pos0 = %lld out of range", static_cast<long long>(pos0));
  if (shape->T == 0) return ok();
  MOE_TRY(need(h_inout, "h_inout"));
  MOE_TRY(need(gamma, "gamma"));
  MOE_TRY(need(wqkv, "wqkv"));
  MOE_TRY(need(wo, "wo"));
  MOE_TRY(need(ws, "ws"));
  const AttnLayout L = attn_layout(shape);
  if (ws_bytes < L.total) return fail(MOE_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", ws_bytes, L.total);
  const int64_t T = shape->T;
  const int d = shape->d, H = shape->H, G = shape->G, dh = shape->d_h;
  const int nqkv = (H + 2 * G) * dh, nq = H * dh;
  int32_t* off = at<int32_t>(ws, L.offsets);
  uint16_t* xn = at<uint16_t>(ws, L.xn);
  float* qkv = at<float>(ws, L.qkv);
  uint16_t* q = at<uint16_t>(ws, L.q);
  uint16_t* k = at<uint16_t>(ws, L.k);
  uint16_t* v = at<uint16_t>(ws, L.v);
  uint16_t* o = at<uint16_t>(ws, L.o);
  float* oproj = at<float>(ws, L.oproj);
  uint16_t* h = static_cast<uint16_t*>(h_inout);
  const hipStream_t st = hs(stream);
  // The projections run on the experts' GEMM as a single expert owning all T
  // rows: the RMSNorm kernel writes those offsets, [0, T], into `off`.
  float* part = L.part < L.total ? at<float>(ws, L.part) : nullptr;
  if (!moe::stream_supported(T, nqkv, d)) {
    // GEMM path: RoPE and the split into q, k, v run in the projection's epilogue.
    float* cs = at<float>(ws, L.cs);
    MOE_TRY(hip_status(moe::launch_rmsnorm_rows(h, gamma, eps, xn, T, d, off, st, cs, static_cast<double>(rope_theta),
                                                pos0),
                       "rmsnorm launch"));
    MOE_TRY(hip_status(moe::launch_gemm_qkv_rope_bf16(xn, off, static_cast<const uint16_t*>(wqkv), cs, q, k, v, T,
                                                      nq, G * dh, d, part, st),
                       "qkv projection launch"));
  } else {
    MOE_TRY(hip_status(moe::launch_rmsnorm_rows(h, gamma, eps, xn, T, d, off, st), "rmsnorm launch"));
    MOE_TRY(hip_status(moe::launch_expert_down_bf16(xn, off, static_cast<const uint16_t*>(wqkv), nullptr, qkv, T, 1,
                                                    nqkv, d, 1, part, st),
                       "qkv projection launch"));
    MOE_TRY(hip_status(moe::launch_rope_pack(qkv, q, k, v, T, H, G, dh, static_cast<double>(rope_theta), pos0, st),
                       "rope launch"));
  }
  MOE_TRY(hip_status(moe::launch_flash_attn(q, k, v, o, T, H, G, dh, st), "attention launch"));
  // On the GEMM path the residual add runs in the projection's epilogue; the
  // streaming path (a few tokens) writes fp32 and adds it after.
  if (!moe::stream_supported(T, d, nq))
    return hip_status(moe::launch_gemm_down_residual_bf16(o, off, static_cast<const uint16_t*>(wo), nullptr, h, T, d,
                                                          nq, 1, part, st),
                      "output projection launch");
  MOE_TRY(hip_status(moe::launch_expert_down_bf16(o, off, static_cast<const uint16_t*>(wo), nullptr, oproj, T, 1, d,
                                                  nq, 1, part, st),
                     "output projection launch"));
  return hip_status(moe::launch_residual_add(h, oproj, T * d, st), "residual launch");
}

moe_status moe_set_timing_events(void* const* events, int32_t count) {
  if (events == nullptr || count == 0) {
    g_timing = false;
    return ok();
  }
  if (count != MOE_TIMING_POINTS)
    return fail(MOE_ERR_INVALID_ARG, "count = %d, expected %d timing events", count, MOE_TIMING_POINTS);
  for (int i = 0; i < MOE_TIMING_POINTS; ++i) {
    if (events[i] == nullptr) return fail(MOE_ERR_INVALID_ARG, "timing event %d is NULL", i);
    g_events[i] = static_cast<hipEvent_t>(events[i]);
  }
  g_timing = true;
  return ok();
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
