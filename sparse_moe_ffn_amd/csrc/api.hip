// libmobmoe C ABI: argument checks on the host, then kernel launches on the
// caller's stream.  See include/mobmoe.h for the contract of every call.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "../../include/mobmoe.h"
#include "launch.h"
#include "launch_train.h"

namespace {

thread_local char g_err[512] = "";

mm_status fail(mm_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

mm_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MM_OK;
  snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
  return MM_ERR_HIP;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define MM_REQUIRE(p)                                                          \
  do {                                                                         \
    if (!(p)) return fail(MM_ERR_NULL, "%s is NULL", #p);                \
    if (!aligned(p)) return fail(MM_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

#define MM_OPTIONAL(p)                                                         \
  do {                                                                         \
    if ((p) && !aligned(p)) return fail(MM_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
  } while (0)

constexpr int64_t kMaxSlots = int64_t(1) << 24;

mm_status check_desc(const mm_layer_desc* d) {
  if (!d) return fail(MM_ERR_NULL, "desc is NULL");
  if (d->d_model < 64 || d->d_model % 64)
    return fail(MM_ERR_SHAPE, "d_model %lld must be a positive multiple of 64", (long long)(d->d_model));
  if (d->n_experts < 1 || d->n_experts > 64)
    return fail(MM_ERR_SHAPE, "n_experts %lld must be in [1, 64]", (long long)(d->n_experts));
  if (d->hidden < 64 || d->hidden % 64)
    return fail(MM_ERR_SHAPE, "hidden %lld must be a positive multiple of 64", (long long)(d->hidden));
  if (d->shared_hidden < 0 || d->shared_hidden % 64)
    return fail(MM_ERR_SHAPE, "shared_hidden %lld must be 0 or a multiple of 64",
                (long long)d->shared_hidden);
  if (d->top_k < 1 || d->top_k > 8 || d->top_k > d->n_experts)
    return fail(MM_ERR_SHAPE, "top_k %lld must be in [1, min(8, n_experts)]", (long long)(d->top_k));
  if (d->wfmt < MM_W_F32 || d->wfmt > MM_W_BF16)
    return fail(MM_ERR_FORMAT, "unknown weight format %lld", (long long)(d->wfmt));
  if (d->gating < 0 || d->gating > (MM_GATE_SIGMOID_NORM | MM_GATE_BIAS_SELECT_ONLY))
    return fail(MM_ERR_FORMAT, "unknown gating rule %lld", (long long)(d->gating));
  if (d->out_dtype < MM_OUT_F32 || d->out_dtype > MM_OUT_BF16)
    return fail(MM_ERR_FORMAT, "unknown output dtype %lld", (long long)(d->out_dtype));
  return MM_OK;
}

mm_status check_T(const mm_layer_desc* d, int64_t T) {
  if (T < 0) return fail(MM_ERR_SHAPE, "T %lld is negative", (long long)(T));
  if (T * d->top_k > kMaxSlots) return fail(MM_ERR_SHAPE, "T*k %lld exceeds 2^24", (long long)(T * d->top_k));
  return MM_OK;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Shared-expert workspace carve-up.
struct SharedWs {
  size_t a_off, q_off, s_off, total;
};
SharedWs shared_ws(const mm_layer_desc* d, int64_t T) {
  SharedWs w{};
  const int64_t hs = d->shared_hidden;
  if (d->wfmt == MM_W_INT4G32) {
    w.a_off = 0;
    w.q_off = align256(T * hs * 4);
    w.s_off = w.q_off + align256(T * hs);
    w.total = w.s_off + align256(T * 4);
  } else if (d->wfmt == MM_W_BF16) {
    w.a_off = 0;                               // BF16 hidden rows
    w.q_off = align256(T * hs * 2);            // BF16 copy of x
    w.total = w.q_off + align256(T * (int64_t)d->d_model * 2);
  } else {
    w.a_off = 0;
    w.total = align256(T * hs * 4);
  }
  return w;
}

// mm_moe_forward workspace carve-up.
struct FwdWs {
  size_t off, perm, inv, route, xq, sx, xb, a_r, q_r, s_r, f, a_s, q_s, s_s, ys, total;
};
FwdWs fwd_ws(const mm_layer_desc* d, int64_t T) {
  const int64_t Tk = T * d->top_k, h = d->hidden, hs = d->shared_hidden, dm = d->d_model;
  const bool i4 = d->wfmt == MM_W_INT4G32, bf = d->wfmt == MM_W_BF16;
  const int64_t hb = i4 ? 4 : (bf ? 2 : 4);  // bytes per hidden value before the down product
  FwdWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  w.off = take((size_t)(d->n_experts + 1) * 4);
  w.perm = take((size_t)Tk * 4);
  w.inv = take((size_t)Tk * 4);
  w.route = take(std::max((size_t)mm::route_blocks(Tk) * d->n_experts * 4,
                          (size_t)d->n_experts * (size_t)mm::route_hist_stride(T)));
  w.xq = take(i4 ? (size_t)T * dm : 0);
  w.sx = take(i4 ? (size_t)T * 4 : 0);
  w.xb = take(bf ? (size_t)T * dm * 2 : 0);
  w.a_r = take((size_t)Tk * h * hb);
  w.q_r = take(i4 ? (size_t)Tk * h : 0);
  w.s_r = take(i4 ? (size_t)Tk * 4 : 0);
  w.f = take((size_t)Tk * dm * 4);
  w.a_s = take((size_t)T * hs * hb);
  w.q_s = take(i4 ? (size_t)T * hs : 0);
  w.s_s = take(i4 ? (size_t)T * 4 : 0);
  w.ys = take(hs ? (size_t)T * dm * 4 : 0);
  w.total = o;
  return w;
}

// mm_moe_decode workspace carve-up: the state block first, then the
// intermediates sized for 4 tokens (the same layout serves every T <= 4).
constexpr int64_t kDecodeMaxT = 4;
struct DecWs {
  size_t state, a_r, a_s, f, ys, total;
};
DecWs dec_ws(const mm_layer_desc* d) {
  const int64_t T = kDecodeMaxT, Tk = T * d->top_k, dm = d->d_model;
  DecWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  // the hand-off buffers hold 8 bytes per value (value and call tag)
  w.state = take(mm::decode_fused_state_bytes());
  w.a_r = take((size_t)Tk * d->hidden * 8);
  w.a_s = take((size_t)T * d->shared_hidden * 8);
  w.f = take((size_t)Tk * dm * 8);
  w.ys = take((size_t)T * dm * 8);
  w.total = o;
  return w;
}
bool decode_applies(const mm_layer_desc* d, int64_t T) {
  return d->wfmt == MM_W_INT4G32 &&
         mm::decode_fused_fits(T, d->d_model, d->n_experts, d->top_k, d->hidden, d->shared_hidden);
}

size_t ws_bytes(const mm_layer_desc* d, int64_t T, int32_t which) {
  const int64_t Tk = T * d->top_k;
  switch (which) {
    case MM_WS_ROUTE:
      return align256((size_t)mm::route_blocks(Tk) * d->n_experts * 4);
    case MM_WS_GATEUP:
      if (d->wfmt == MM_W_INT4G32) return align256((size_t)Tk * d->hidden * 4);
      if (d->wfmt == MM_W_BF16) return align256((size_t)T * d->d_model * 2);  // BF16 copy of x
      return 0;
    case MM_WS_DOWN:
      return 0;
    case MM_WS_SHARED:
      return d->shared_hidden ? shared_ws(d, T).total : 0;
    case MM_WS_MAX: {
      size_t m = 0;
      for (int i = 0; i < MM_WS_MAX; ++i) m = std::max(m, ws_bytes(d, T, i));
      return m;
    }
    case MM_WS_FORWARD:
      return fwd_ws(d, T).total;
    case MM_WS_DECODE:
      return decode_applies(d, std::max<int64_t>(T, 1)) ? dec_ws(d).total : 0;
    default:
      return 0;
  }
}

mm_status check_weight(const mm_layer_desc* d, const mm_weight& w, const char* name) {
  if (!w.data) return fail(MM_ERR_NULL, "%s.data is NULL", name);
  if (!aligned(w.data)) return fail(MM_ERR_ALIGN, "%s.data is not 16-byte aligned", name);
  if (d->wfmt == MM_W_INT4G32) {
    if (!w.scales) return fail(MM_ERR_NULL, "%s.scales is NULL for INT4 weights", name);
    if (!aligned(w.scales)) return fail(MM_ERR_ALIGN, "%s.scales is not 16-byte aligned", name);
  } else if (w.scales) {
    return fail(MM_ERR_FORMAT, "%s.scales must be NULL for non-INT4 weights", name);
  }
  return MM_OK;
}

#define MM_TRY(expr)                 \
  do {                               \
    mm_status _s = (expr);           \
    if (_s != MM_OK) return _s;      \
  } while (0)

hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

// INT4 products.  Few rows per expert: the weight-streaming kernels (decode).
// Otherwise the matrix-core kernels.  The gate/up of both writes the FP32
// hidden rows to abuf, then the row quantiser produces hq / hs.  Shapes
// neither supports go to the row-tile kernels, whose gate/up quantises in
// place.
bool use_gemv(const mm::ExpertArgs& a, int K, bool gateup) {
  const int64_t lim = a.offsets ? mm::kGemvMaxRowsRouted : mm::kGemvMaxRowsDense;
  return a.rows <= lim && mm::gemv_i4_fits(K, gateup);
}

// Matrix cores: routed from 256 rows; dense (shared expert) beyond the
// weight-streaming range.
bool use_mfma(const mm::ExpertArgs& a, int K) {
  const int64_t lo = a.offsets ? mm::kMfmaMinRows : mm::kGemvMaxRowsDense + 1;
  return a.rows >= lo && K % mm::kMfmaK == 0;
}

// hq == nullptr: the FP32 rows in abuf are the output (no re-quantisation).
hipError_t gateup_i4(const mm::ExpertArgs& a, const int8_t* xq, const float* sx,
                     const uint8_t* wq, const float* ws, float* abuf, int8_t* hq, float* hs,
                     int32_t* isum, hipStream_t st) {
  hipError_t e;
  if (use_gemv(a, a.d, true))
    e = mm::launch_gateup_i4_gemv(a, xq, sx, wq, ws, abuf, isum, st);
  else if (use_mfma(a, a.d))
    e = mm::launch_gateup_i4_mfma(a, xq, sx, wq, ws, abuf, isum, st);
  else
    return mm::launch_gateup_i4(a, xq, sx, wq, ws, abuf, hq, hs, isum, st);
  if (e != hipSuccess || hq == nullptr) return e;
  return mm::launch_act_quant_i8(a.rows, a.h, abuf, hq, hs, st);
}

hipError_t down_i4(const mm::ExpertArgs& a, const int8_t* hq, const float* hs,
                   const uint8_t* wq, const float* ws, float* f, int32_t* isum, hipStream_t st) {
  if (use_gemv(a, a.h, false)) return mm::launch_down_i4_gemv(a, hq, hs, wq, ws, f, isum, st);
  if (use_mfma(a, a.h)) return mm::launch_down_i4_mfma(a, hq, hs, wq, ws, f, isum, st);
  return mm::launch_down_i4(a, hq, hs, wq, ws, f, isum, st);
}

}  // namespace

namespace {

// mm_moe_decode and mm_moe_decode_noalloc: every check, then the launch on
// the workspace from get_ws(needed bytes, &base) (called after the checks).
template <class GetWs>
mm_status moe_decode_impl(const char* where, const mm_layer_desc* desc, int64_t T, const float* x,
                          const float* w_router, const float* bias, mm_weight w_gateup,
                          mm_weight w_down, mm_weight ws_gateup, mm_weight ws_down,
                          int32_t* topk_idx, float* topk_w, void* y, float* y_norm, float norm_eps,
                          void* stream, const GetWs& get_ws) {
  MM_TRY(check_desc(desc));
  if (T < 0) return fail(MM_ERR_SHAPE, "T %lld is negative", (long long)T);
  if (T == 0) return MM_OK;
  if (desc->wfmt != MM_W_INT4G32) return fail(MM_ERR_FORMAT, "%s needs INT4 weights", where);
  if (!decode_applies(desc, T))
    return fail(MM_ERR_SHAPE,
                "%s: no one-launch form for T=%lld d=%d h=%d h_s=%d (T <= 4, d %% 128 == 0, "
                "d <= 1280, h and h_s multiples of 128 up to 2560)",
                where, (long long)T, desc->d_model, desc->hidden, desc->shared_hidden);
  MM_REQUIRE(x);
  MM_REQUIRE(w_router);
  MM_OPTIONAL(bias);
  MM_REQUIRE(topk_idx);
  MM_REQUIRE(topk_w);
  MM_REQUIRE(y);
  MM_OPTIONAL(y_norm);
  if (y_norm && desc->out_dtype != MM_OUT_F32)
    return fail(MM_ERR_FORMAT, "y_norm needs FP32 output");
  if (y_norm && !(norm_eps > 0.0f)) return fail(MM_ERR_SHAPE, "norm_eps must be positive");
  MM_TRY(check_weight(desc, w_gateup, "w_gateup"));
  MM_TRY(check_weight(desc, w_down, "w_down"));
  const bool shared = desc->shared_hidden > 0;
  if (shared) {
    MM_TRY(check_weight(desc, ws_gateup, "ws_gateup"));
    MM_TRY(check_weight(desc, ws_down, "ws_down"));
  }
  const DecWs W = dec_ws(desc);
  char* base = nullptr;
  MM_TRY(get_ws(W.total, &base));
  mm::DecodeFusedArgs a{};
  a.T = T;
  a.d = desc->d_model;
  a.E = desc->n_experts;
  a.k = desc->top_k;
  a.h = desc->hidden;
  a.hs = desc->shared_hidden;
  a.gating = desc->gating;
  a.x = x;
  a.wr = w_router;
  a.bias = bias;
  a.gq = static_cast<const uint8_t*>(w_gateup.data);
  a.gs = w_gateup.scales;
  a.dq = static_cast<const uint8_t*>(w_down.data);
  a.ds = w_down.scales;
  a.sgq = shared ? static_cast<const uint8_t*>(ws_gateup.data) : nullptr;
  a.sgs = shared ? ws_gateup.scales : nullptr;
  a.sdq = shared ? static_cast<const uint8_t*>(ws_down.data) : nullptr;
  a.sds = shared ? ws_down.scales : nullptr;
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.y = y;
  a.y_norm = y_norm;
  a.eps = norm_eps;
  a.out_bf16 = desc->out_dtype == MM_OUT_BF16;
  a.state = base + W.state;
  a.a_r = base + W.a_r;
  a.a_s = base + W.a_s;
  a.f = base + W.f;
  a.ys = base + W.ys;
  a.spin_limit = 1u << 20;
  return hip_status(mm::launch_decode_fused(a, S(stream)), where);
}

}  // namespace

extern "C" {

const char* mm_version(void) { return "libmobmoe 0.1 (gfx950)"; }

const char* mm_status_string(mm_status s) {
  switch (s) {
    case MM_OK: return "MM_OK";
    case MM_ERR_NULL: return "MM_ERR_NULL";
    case MM_ERR_SHAPE: return "MM_ERR_SHAPE";
    case MM_ERR_ALIGN: return "MM_ERR_ALIGN";
    case MM_ERR_FORMAT: return "MM_ERR_FORMAT";
    case MM_ERR_WORKSPACE: return "MM_ERR_WORKSPACE";
    case MM_ERR_HIP: return "MM_ERR_HIP";
  }
  return "MM_ERR_UNKNOWN";
}

const char* mm_last_error_string(void) { return g_err; }

size_t mm_workspace_bytes(const mm_layer_desc* desc, int64_t T, int32_t which) {
  if (check_desc(desc) != MM_OK || T < 0) return 0;
  return ws_bytes(desc, T, which);
}

mm_status mm_quantize_int4g32(int64_t rows, int64_t cols, const float* w, uint8_t* q,
                              float* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return fail(MM_ERR_SHAPE, "cols %lld must be a positive multiple of 32", (long long)(cols));
  if (rows == 0) return MM_OK;
  MM_REQUIRE(w);
  MM_REQUIRE(q);
  MM_REQUIRE(scales);
  return hip_status(mm::launch_quantize_int4g32(rows, cols, w, q, scales, S(stream)),
                    "mm_quantize_int4g32");
}

size_t mm_prepacked_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || rows % 32 || cols % 32) return 0;
  return (size_t)rows * cols / 2;
}

size_t mm_prepacked_scale_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || rows % 32 || cols % 32) return 0;
  return (size_t)rows * (cols / 32) * 4;
}

mm_status mm_prepack_int4g32(int64_t n_mat, int64_t rows, int64_t cols, const uint8_t* q_canon,
                             const float* s_canon, uint8_t* q_out, float* s_out, void* stream) {
  if (n_mat < 0 || rows <= 0 || cols <= 0 || rows % 32 || cols % 32)
    return fail(MM_ERR_SHAPE, "prepack needs rows and cols multiples of 32");
  if (n_mat == 0) return MM_OK;
  MM_REQUIRE(q_canon);
  MM_REQUIRE(s_canon);
  MM_REQUIRE(q_out);
  MM_REQUIRE(s_out);
  return hip_status(mm::launch_prepack_int4g32(n_mat, rows, cols, q_canon, s_canon, q_out, s_out,
                                               S(stream)),
                    "mm_prepack_int4g32");
}

mm_status mm_convert_bf16(int64_t n, const float* x, uint16_t* y, void* stream) {
  if (n < 0) return fail(MM_ERR_SHAPE, "n %lld is negative", (long long)(n));
  if (n == 0) return MM_OK;
  MM_REQUIRE(x);
  MM_REQUIRE(y);
  return hip_status(mm::launch_convert_bf16(n, x, y, S(stream)), "mm_convert_bf16");
}

mm_status mm_router_topk(const mm_layer_desc* desc, int64_t T, const float* x,
                         const float* w_router, const float* bias, int32_t* topk_idx,
                         float* topk_w, void* stream) {
  MM_TRY(check_desc(desc));
  MM_TRY(check_T(desc, T));
  if (T == 0) return MM_OK;
  MM_REQUIRE(x);
  MM_REQUIRE(w_router);
  MM_OPTIONAL(bias);
  MM_REQUIRE(topk_idx);
  MM_REQUIRE(topk_w);
  return hip_status(mm::launch_router(T, desc->d_model, desc->n_experts, desc->top_k, desc->gating,
                                      x, w_router, bias, topk_idx, topk_w, nullptr, nullptr,
                                      S(stream)),
                    "mm_router_topk");
}

mm_status mm_route_permute(const mm_layer_desc* desc, int64_t T, const int32_t* topk_idx,
                           int32_t* expert_offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                           size_t ws_size, void* stream) {
  MM_TRY(check_desc(desc));
  MM_TRY(check_T(desc, T));
  if (T == 0) return MM_OK;
  MM_REQUIRE(topk_idx);
  MM_REQUIRE(expert_offsets);
  MM_REQUIRE(perm);
  MM_REQUIRE(inv_perm);
  MM_REQUIRE(ws);
  if (ws_size < ws_bytes(desc, T, MM_WS_ROUTE))
    return fail(MM_ERR_WORKSPACE, "route workspace too small (need %lld bytes)", (long long)ws_bytes(desc, T, MM_WS_ROUTE));
  return hip_status(mm::launch_route(T * desc->top_k, desc->n_experts, topk_idx, expert_offsets,
                                     perm, inv_perm, static_cast<int32_t*>(ws), S(stream)),
                    "mm_route_permute");
}

mm_status mm_act_quant_i8(int64_t rows, int64_t cols, const float* x, int8_t* q, float* scale,
                          void* stream) {
  if (rows < 0 || cols <= 0) return fail(MM_ERR_SHAPE, "bad shape");
  if (rows == 0) return MM_OK;
  MM_REQUIRE(x);
  MM_REQUIRE(q);
  MM_REQUIRE(scale);
  return hip_status(mm::launch_act_quant_i8(rows, cols, x, q, scale, S(stream)), "mm_act_quant_i8");
}

static mm_status gateup_impl(const mm_layer_desc* desc, int64_t T, const void* act,
                             const float* act_scale, const int32_t* perm,
                             const int32_t* expert_offsets, mm_weight w, void* h, float* h_scale,
                             void* ws, size_t ws_size, int32_t* isum, void* stream) {
  MM_TRY(check_desc(desc));
  MM_TRY(check_T(desc, T));
  if (T == 0) return MM_OK;
  MM_REQUIRE(act);
  MM_REQUIRE(perm);
  MM_REQUIRE(expert_offsets);
  MM_REQUIRE(h);
  MM_TRY(check_weight(desc, w, "w_gateup"));
  mm::ExpertArgs a{T * desc->top_k, T, desc->d_model, desc->hidden, desc->n_experts, desc->top_k,
                   perm, expert_offsets};
  hipStream_t st = S(stream);
  if (desc->wfmt == MM_W_INT4G32) {
    MM_REQUIRE(act_scale);
    if (h_scale == nullptr)  // FP32 hidden rows straight into h
      return hip_status(gateup_i4(a, static_cast<const int8_t*>(act), act_scale,
                                  static_cast<const uint8_t*>(w.data), w.scales,
                                  static_cast<float*>(h), nullptr, nullptr, isum, st),
                        "mm_expert_gateup_swiglu");
    MM_REQUIRE(ws);
    if (ws_size < ws_bytes(desc, T, MM_WS_GATEUP))
      return fail(MM_ERR_WORKSPACE, "gate/up workspace too small (need %lld bytes)", (long long)ws_bytes(desc, T, MM_WS_GATEUP));
    float* abuf = static_cast<float*>(ws);
    return hip_status(gateup_i4(a, static_cast<const int8_t*>(act), act_scale,
                                static_cast<const uint8_t*>(w.data), w.scales, abuf,
                                static_cast<int8_t*>(h), h_scale, isum, st),
                      "mm_expert_gateup_swiglu");
  }
  if (act_scale || h_scale)
    return fail(MM_ERR_FORMAT, "act_scale and h_scale must be NULL for FP32/BF16 weights");
  if (desc->wfmt == MM_W_BF16) {  // x rounded to BF16 once, then the bf16 matrix cores
    MM_REQUIRE(ws);
    if (ws_size < ws_bytes(desc, T, MM_WS_GATEUP))
      return fail(MM_ERR_WORKSPACE, "gate/up workspace too small (need %lld bytes)", (long long)ws_bytes(desc, T, MM_WS_GATEUP));
    uint16_t* xb = static_cast<uint16_t*>(ws);
    MM_TRY(hip_status(mm::launch_convert_bf16(T * desc->d_model, static_cast<const float*>(act), xb, st),
                      "mm_expert_gateup_swiglu"));
    return hip_status(mm::launch_gateup_bf16_mfma(a, xb, static_cast<const uint16_t*>(w.data),
                                                  static_cast<uint16_t*>(h), st),
                      "mm_expert_gateup_swiglu");
  }
  return hip_status(mm::launch_gateup_fp(a, false, act, w.data, h, st), "mm_expert_gateup_swiglu");
}

mm_status mm_act_quant_i8_layout(int64_t rows, int64_t cols, const float* x, int8_t* q,
                                 float* scale, int32_t layout, void* stream) {
  if (layout != MM_ACT_ROW_MAJOR && layout != MM_ACT_GROUP_MAJOR && layout != MM_ACT_F16_PAIRED)
    return fail(MM_ERR_FORMAT, "unknown activation layout %d", (int)layout);
  if (rows < 0 || cols <= 0) return fail(MM_ERR_SHAPE, "bad shape");
  if (layout != MM_ACT_ROW_MAJOR && cols % 128 != 0)
    return fail(MM_ERR_SHAPE, "group-major and f16 paired codes need cols %% 128 == 0");
  if (rows == 0) return MM_OK;
  MM_REQUIRE(x);
  MM_REQUIRE(q);
  MM_REQUIRE(scale);
  const int lay = layout == MM_ACT_GROUP_MAJOR ? mm::kActGroupMajor
                  : layout == MM_ACT_F16_PAIRED ? mm::kActF16Paired
                                                : mm::kActRowMajor;
  return hip_status(mm::launch_act_quant_i8(rows, cols, x, q, scale, S(stream), lay),
                    "mm_act_quant_i8_layout");
}

namespace {

// Checks shared by the merged product entries: INT4 weights, a shared
// expert, and widths the f16 matrix-core products take.
mm_status check_pair(const mm_layer_desc* desc, int64_t T, const char* what) {
  MM_TRY(check_desc(desc));
  MM_TRY(check_T(desc, T));
  if (desc->wfmt != MM_W_INT4G32) return fail(MM_ERR_FORMAT, "the merged %s takes INT4 weights", what);
  if (desc->shared_hidden <= 0) return fail(MM_ERR_SHAPE, "the merged %s needs a shared expert", what);
  if (!mm::f16_products_fit(desc->d_model, desc->hidden, desc->shared_hidden))
    return fail(MM_ERR_SHAPE, "the merged %s needs d %% 128 == 0 and h, h_s %% 64 == 0", what);
  return MM_OK;
}

mm_status gateup_pair_impl(const mm_layer_desc* desc, int64_t T, const void* xq, const float* sx,
                           const int32_t* perm, const int32_t* expert_offsets, mm_weight w_gateup,
                           mm_weight ws_gateup, float* h_r, float* h_s, int32_t* isum_r,
                           int32_t* isum_s, void* stream, const char* where) {
  MM_TRY(check_pair(desc, T, "gate/up"));
  if (T == 0) return MM_OK;
  MM_REQUIRE(xq);
  MM_REQUIRE(sx);
  MM_REQUIRE(perm);
  MM_REQUIRE(expert_offsets);
  MM_REQUIRE(h_r);
  MM_REQUIRE(h_s);
  MM_TRY(check_weight(desc, w_gateup, "w_gateup"));
  MM_TRY(check_weight(desc, ws_gateup, "ws_gateup"));
  const int k = desc->top_k;
  const mm::ExpertArgs ar{T * k, T, desc->d_model, desc->hidden, desc->n_experts, k, perm,
                          expert_offsets};
  const mm::ExpertArgs as{T, T, desc->d_model, desc->shared_hidden, 1, 1, nullptr, nullptr};
  return hip_status(mm::launch_gateup_f16_pair(
                        ar, as, static_cast<const uint16_t*>(xq), sx,
                        static_cast<const uint8_t*>(w_gateup.data), w_gateup.scales,
                        static_cast<const uint8_t*>(ws_gateup.data), ws_gateup.scales, h_r, h_s,
                        isum_r, isum_s, S(stream)),
                    where);
}

mm_status down_pair_impl(const mm_layer_desc* desc, int64_t T, const void* hq_r,
                         const float* hs_r, const void* hq_s, const float* hs_s,
                         const int32_t* expert_offsets, mm_weight w_down, mm_weight ws_down,
                         float* f, float* ys, int32_t* isum_r, int32_t* isum_s, void* stream,
                         const char* where) {
  MM_TRY(check_pair(desc, T, "down"));
  if (T == 0) return MM_OK;
  MM_REQUIRE(hq_r);
  MM_REQUIRE(hs_r);
  MM_REQUIRE(hq_s);
  MM_REQUIRE(hs_s);
  MM_REQUIRE(expert_offsets);
  MM_REQUIRE(f);
  MM_REQUIRE(ys);
  MM_TRY(check_weight(desc, w_down, "w_down"));
  MM_TRY(check_weight(desc, ws_down, "ws_down"));
  const int k = desc->top_k;
  const mm::ExpertArgs ar{T * k, T, desc->d_model, desc->hidden, desc->n_experts, k, nullptr,
                          expert_offsets};
  const mm::ExpertArgs as{T, T, desc->d_model, desc->shared_hidden, 1, 1, nullptr, nullptr};
  return hip_status(mm::launch_down_f16_pair(
                        ar, as, static_cast<const uint16_t*>(hq_r), hs_r,
                        static_cast<const uint16_t*>(hq_s), hs_s,
                        static_cast<const uint8_t*>(w_down.data), w_down.scales,
                        static_cast<const uint8_t*>(ws_down.data), ws_down.scales, f, ys, isum_r,
                        isum_s, S(stream)),
                    where);
}

}  // namespace

mm_status mm_expert_gateup_pair_f32(const mm_layer_desc* desc, int64_t T, const void* xq,
                                    const float* sx, const int32_t* perm,
                                    const int32_t* expert_offsets, mm_weight w_gateup,
                                    mm_weight ws_gateup, float* h_r, float* h_s, void* stream) {
  return gateup_pair_impl(desc, T, xq, sx, perm, expert_offsets, w_gateup, ws_gateup, h_r, h_s,
                          nullptr, nullptr, stream, "mm_expert_gateup_pair_f32");
}

mm_status mm_expert_gateup_pair_f32_dbg(const mm_layer_desc* desc, int64_t T, const void* xq,
                                        const float* sx, const int32_t* perm,
                                        const int32_t* expert_offsets, mm_weight w_gateup,
                                        mm_weight ws_gateup, float* h_r, float* h_s,
                                        int32_t* isum_r, int32_t* isum_s, void* stream) {
  MM_REQUIRE(isum_r);
  MM_REQUIRE(isum_s);
  return gateup_pair_impl(desc, T, xq, sx, perm, expert_offsets, w_gateup, ws_gateup, h_r, h_s,
                          isum_r, isum_s, stream, "mm_expert_gateup_pair_f32_dbg");
}

mm_status mm_expert_down_pair_f32(const mm_layer_desc* desc, int64_t T, const void* hq_r,
                                  const float* hs_r, const void* hq_s, const float* hs_s,
                                  const int32_t* expert_offsets, mm_weight w_down,
                                  mm_weight ws_down, float* f, float* ys, void* stream) {
  return down_pair_impl(desc, T, hq_r, hs_r, hq_s, hs_s, expert_offsets, w_down, ws_down, f, ys,
                        nullptr, nullptr, stream, "mm_expert_down_pair_f32");
}

mm_status mm_expert_down_pair_f32_dbg(const mm_layer_desc* desc, int64_t T, const void* hq_r,
                                      const float* hs_r, const void* hq_s, const float* hs_s,
                                      const int32_t* expert_offsets, mm_weight w_down,
                                      mm_weight ws_down, float* f, float* ys, int32_t* isum_r,
                                      int32_t* isum_s, void* stream) {
  MM_REQUIRE(isum_r);
  MM_REQUIRE(isum_s);
  return down_pair_impl(desc, T, hq_r, hs_r, hq_s, hs_s, expert_offsets, w_down, ws_down, f, ys,
                        isum_r, isum_s, stream, "mm_expert_down_pair_f32_dbg");
}

mm_status mm_expert_gateup_swiglu(const mm_layer_desc* desc, int64_t T, const void* act,
                                  const float* act_scale, const int32_t* perm,
                                  const int32_t* expert_offsets, mm_weight w_gateup, void* h,
                                  float* h_scale, void* ws, size_t ws_size, void* stream) {
  return gateup_impl(desc, T, act, act_scale, perm, expert_offsets, w_gateup, h, h_scale, ws,
                     ws_size, nullptr, stream);
}

mm_status mm_expert_gateup_swiglu_dbg(const mm_layer_desc* desc, int64_t T, const void* act,
                                      const float* act_scale, const int32_t* perm,
                                      const int32_t* expert_offsets, mm_weight w_gateup,
                                      void* h, float* h_scale, void* ws, size_t ws_size,
                                      int32_t* isum, void* stream) {
  if (desc && desc->wfmt != MM_W_INT4G32)
    return fail(MM_ERR_FORMAT, "group sums exist only for INT4 weights");
  MM_REQUIRE(isum);
  return gateup_impl(desc, T, act, act_scale, perm, expert_offsets, w_gateup, h, h_scale, ws,
                     ws_size, isum, stream);
}

static mm_status down_impl(const mm_layer_desc* desc, int64_t T, const void* h,
                           const float* h_scale, const int32_t* expert_offsets, mm_weight w,
                           float* f, int32_t* isum, void* stream) {
  MM_TRY(check_desc(desc));
  MM_TRY(check_T(desc, T));
  if (T == 0) return MM_OK;
  MM_REQUIRE(h);
  MM_REQUIRE(expert_offsets);
  MM_REQUIRE(f);
  MM_TRY(check_weight(desc, w, "w_down"));
  mm::ExpertArgs a{T * desc->top_k, T, desc->d_model, desc->hidden, desc->n_experts, desc->top_k,
                   nullptr, expert_offsets};
  hipStream_t st = S(stream);
  if (desc->wfmt == MM_W_INT4G32) {
    MM_REQUIRE(h_scale);
    return hip_status(down_i4(a, static_cast<const int8_t*>(h), h_scale,
                              static_cast<const uint8_t*>(w.data), w.scales, f, isum, st),
                      "mm_expert_down");
  }
  if (h_scale) return fail(MM_ERR_FORMAT, "h_scale must be NULL for FP32/BF16 weights");
  if (desc->wfmt == MM_W_BF16)
    return hip_status(mm::launch_down_bf16_mfma(a, static_cast<const uint16_t*>(h),
                                                static_cast<const uint16_t*>(w.data), f, st),
                      "mm_expert_down");
  return hip_status(mm::launch_down_fp(a, false, h, w.data, f, st), "mm_expert_down");
}

mm_status mm_expert_down(const mm_layer_desc* desc, int64_t T, const void* h,
                         const float* h_scale, const int32_t* expert_offsets, mm_weight w_down,
                         float* f, void* ws, size_t ws_size, void* stream) {
  (void)ws;
  (void)ws_size;
  return down_impl(desc, T, h, h_scale, expert_offsets, w_down, f, nullptr, stream);
}

mm_status mm_expert_down_dbg(const mm_layer_desc* desc, int64_t T, const void* h,
                             const float* h_scale, const int32_t* expert_offsets,
                             mm_weight w_down, float* f, void* ws, size_t ws_size,
                             int32_t* isum, void* stream) {
  (void)ws;
  (void)ws_size;
  if (desc && desc->wfmt != MM_W_INT4G32)
    return fail(MM_ERR_FORMAT, "group sums exist only for INT4 weights");
  MM_REQUIRE(isum);
  return down_impl(desc, T, h, h_scale, expert_offsets, w_down, f, isum, stream);
}

mm_status mm_shared_expert(const mm_layer_desc* desc, int64_t T, const void* act,
                           const float* act_scale, mm_weight w_gateup, mm_weight w_down,
                           float* ys, void* ws, size_t ws_size, void* stream) {
  MM_TRY(check_desc(desc));
  MM_TRY(check_T(desc, T));
  if (desc->shared_hidden == 0) return fail(MM_ERR_SHAPE, "no shared expert (shared_hidden == 0)");
  if (T == 0) return MM_OK;
  MM_REQUIRE(act);
  MM_REQUIRE(ys);
  MM_REQUIRE(ws);
  MM_TRY(check_weight(desc, w_gateup, "w_gateup"));
  MM_TRY(check_weight(desc, w_down, "w_down"));
  const SharedWs sw = shared_ws(desc, T);
  if (ws_size < sw.total)
    return fail(MM_ERR_WORKSPACE, "shared workspace too small (need %lld bytes)", (long long)sw.total);
  mm::ExpertArgs a{T, T, desc->d_model, desc->shared_hidden, 1, 1, nullptr, nullptr};
  hipStream_t st = S(stream);
  char* base = static_cast<char*>(ws);
  if (desc->wfmt == MM_W_INT4G32) {
    MM_REQUIRE(act_scale);
    float* abuf = reinterpret_cast<float*>(base + sw.a_off);
    int8_t* hq = reinterpret_cast<int8_t*>(base + sw.q_off);
    float* hsc = reinterpret_cast<float*>(base + sw.s_off);
    MM_TRY(hip_status(gateup_i4(a, static_cast<const int8_t*>(act), act_scale,
                                static_cast<const uint8_t*>(w_gateup.data), w_gateup.scales,
                                abuf, hq, hsc, nullptr, st),
                      "mm_shared_expert (gate/up)"));
    return hip_status(down_i4(a, hq, hsc, static_cast<const uint8_t*>(w_down.data),
                              w_down.scales, ys, nullptr, st),
                      "mm_shared_expert (down)");
  }
  if (act_scale) return fail(MM_ERR_FORMAT, "act_scale must be NULL for FP32/BF16 weights");
  void* hbuf = base + sw.a_off;
  if (desc->wfmt == MM_W_BF16) {
    uint16_t* xb = reinterpret_cast<uint16_t*>(base + sw.q_off);
    MM_TRY(hip_status(mm::launch_convert_bf16(T * desc->d_model, static_cast<const float*>(act), xb, st),
                      "mm_shared_expert (x to BF16)"));
    MM_TRY(hip_status(mm::launch_gateup_bf16_mfma(a, xb, static_cast<const uint16_t*>(w_gateup.data),
                                                  static_cast<uint16_t*>(hbuf), st),
                      "mm_shared_expert (gate/up)"));
    return hip_status(mm::launch_down_bf16_mfma(a, static_cast<const uint16_t*>(hbuf),
                                                static_cast<const uint16_t*>(w_down.data), ys, st),
                      "mm_shared_expert (down)");
  }
  MM_TRY(hip_status(mm::launch_gateup_fp(a, false, act, w_gateup.data, hbuf, st),
                    "mm_shared_expert (gate/up)"));
  return hip_status(mm::launch_down_fp(a, false, hbuf, w_down.data, ys, st), "mm_shared_expert (down)");
}

mm_status mm_combine(const mm_layer_desc* desc, int64_t T, const float* f,
                     const int32_t* inv_perm, const float* topk_w, const float* ys, void* y,
                     void* stream) {
  MM_TRY(check_desc(desc));
  MM_TRY(check_T(desc, T));
  if (T == 0) return MM_OK;
  MM_REQUIRE(f);
  MM_REQUIRE(inv_perm);
  MM_REQUIRE(topk_w);
  MM_OPTIONAL(ys);
  MM_REQUIRE(y);
  return hip_status(mm::launch_combine(T, desc->d_model, desc->top_k, f, inv_perm, topk_w, ys, y,
                                       desc->out_dtype == MM_OUT_BF16, S(stream)),
                    "mm_combine");
}

static hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;

mm_status mm_set_profile_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(MM_ERR_NULL, "profile events: give both or neither");
  g_prof_start = static_cast<hipEvent_t>(start);
  g_prof_stop = static_cast<hipEvent_t>(stop);
  return MM_OK;
}

mm_status mm_moe_forward(const mm_layer_desc* desc, int64_t T, const float* x,
                         const float* w_router, const float* bias, mm_weight w_gateup,
                         mm_weight w_down, mm_weight ws_gateup, mm_weight ws_down,
                         int32_t* topk_idx, float* topk_w, void* y, float* y_norm, float norm_eps,
                         void* ws, size_t ws_size, void* stream) {
  MM_TRY(check_desc(desc));
  MM_TRY(check_T(desc, T));
  if (T == 0) return MM_OK;
  MM_REQUIRE(x);
  MM_REQUIRE(w_router);
  MM_OPTIONAL(bias);
  MM_REQUIRE(topk_idx);
  MM_REQUIRE(topk_w);
  MM_REQUIRE(y);
  MM_OPTIONAL(y_norm);
  if (y_norm && desc->out_dtype != MM_OUT_F32)
    return fail(MM_ERR_FORMAT, "y_norm needs FP32 output");
  if (y_norm && !(norm_eps > 0.0f)) return fail(MM_ERR_SHAPE, "norm_eps must be positive");
  MM_REQUIRE(ws);
  MM_TRY(check_weight(desc, w_gateup, "w_gateup"));
  MM_TRY(check_weight(desc, w_down, "w_down"));
  const bool shared = desc->shared_hidden > 0;
  if (shared) {
    MM_TRY(check_weight(desc, ws_gateup, "ws_gateup"));
    MM_TRY(check_weight(desc, ws_down, "ws_down"));
  }
  const FwdWs W = fwd_ws(desc, T);
  if (ws_size < W.total)
    return fail(MM_ERR_WORKSPACE, "forward workspace too small (need %lld bytes)", (long long)W.total);
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  const int d = desc->d_model, E = desc->n_experts, k = desc->top_k;
  const int h = desc->hidden, hs = desc->shared_hidden;
  const int64_t Tk = T * k;
  int32_t* off = static_cast<int32_t*>(at(W.off));
  int32_t* perm = static_cast<int32_t*>(at(W.perm));
  int32_t* inv = static_cast<int32_t*>(at(W.inv));
  float* f = static_cast<float*>(at(W.f));
  float* ys = shared ? static_cast<float*>(at(W.ys)) : nullptr;
  const mm::ExpertArgs ar{Tk, T, d, h, E, k, perm, off};
  const mm::ExpertArgs as{T, T, d, hs, 1, 1, nullptr, nullptr};
  hipStream_t st = S(stream);
  const char* where = "mm_moe_forward";
  const bool i4 = desc->wfmt == MM_W_INT4G32;
  int8_t* xq = i4 ? static_cast<int8_t*>(at(W.xq)) : nullptr;
  float* sx = i4 ? static_cast<float*>(at(W.sx)) : nullptr;

  // Which kernels run (INT4): gate/up and down each as the weight-streaming
  // pair (few rows), the matrix-core pair, or separate launches; both down
  // products streaming from the FP32 hidden rows when both fit (qin).  The
  // matrix-core pairs read group-major activations, so x_q and the hidden
  // codes are written that way when they are used.
  bool gv = false, gm = false, dv = false, dm = false, qin = false;
  bool gu_mfma_pair = false, quant_pair = false, dn_mfma_pair = false;
  if (i4) {
    gv = use_gemv(ar, d, true) && (!shared || use_gemv(as, d, true));
    gm = use_mfma(ar, d) && (!shared || use_mfma(as, d));
    dv = use_gemv(ar, h, false) && (!shared || use_gemv(as, hs, false));
    dm = use_mfma(ar, h) && (!shared || use_mfma(as, hs));
    qin = shared && gv && dv && mm::gemv_i4_qin_fits(h) && mm::gemv_i4_qin_fits(hs);
    gu_mfma_pair = shared && !gv && gm && !use_gemv(ar, d, true);
    quant_pair = (shared && gv && !qin) || gu_mfma_pair;
    dn_mfma_pair = !qin && shared && !dv && dm && !use_gemv(ar, h, false) && quant_pair;
  }
  const int xq_layout = gu_mfma_pair ? mm::kActGroupMajor : mm::kActRowMajor;
  // the matrix-core down pair with FP32 output and no fused RMSNorm: the
  // combine runs in the shared down's epilogue (no ys, no combine launch)
  const bool cmb_in_down = dn_mfma_pair && y_norm == nullptr && desc->out_dtype == MM_OUT_F32 &&
                           mm::down_cmb_fits(ar, as);

  // router + top-k (+ per-token INT8 of x), then the count sort; for a few
  // tokens all of it in one workgroup
  if (i4 && !gu_mfma_pair &&
      mm::launch_front_small(T, d, E, k, desc->gating, x, w_router, bias, topk_idx, topk_w, xq, sx,
                             off, perm, inv, st)) {
    MM_TRY(hip_status(hipGetLastError(), where));
  } else {
    // many tokens: the router also counts the experts of each of its
    // workgroups, and the count sort is one kernel
    const bool hist = mm::route_hist_applies(T, k);
    uint8_t* hbuf = hist ? static_cast<uint8_t*>(at(W.route)) : nullptr;
    MM_TRY(hip_status(mm::launch_router(T, d, E, k, desc->gating, x, w_router, bias, topk_idx,
                                        topk_w, xq, sx, st, xq_layout, hbuf,
                                        hist ? mm::route_hist_stride(T) : 0),
                      where));
    if (hist)
      MM_TRY(hip_status(mm::launch_route_hist(T, k, E, topk_idx, hbuf, off, perm, inv, st), where));
    else
      MM_TRY(hip_status(mm::launch_route(Tk, E, topk_idx, off, perm, inv,
                                         static_cast<int32_t*>(at(W.route)), st),
                        where));
  }
  if (i4) {
    const uint8_t* gq = static_cast<const uint8_t*>(w_gateup.data);
    const uint8_t* dq = static_cast<const uint8_t*>(w_down.data);
    const uint8_t* sgq = static_cast<const uint8_t*>(ws_gateup.data);
    const uint8_t* sdq = static_cast<const uint8_t*>(ws_down.data);
    float* a_r = static_cast<float*>(at(W.a_r));
    float* a_s = static_cast<float*>(at(W.a_s));
    int8_t* q_r = static_cast<int8_t*>(at(W.q_r));
    int8_t* q_s = static_cast<int8_t*>(at(W.q_s));
    float* s_r = static_cast<float*>(at(W.s_r));
    float* s_s = static_cast<float*>(at(W.s_s));
    // gate/up (+ SwiGLU) of both kinds, then their hidden-row quantisers
    // (weight-streaming down of both kinds: the down workgroups quantise)
    if (g_prof_start) MM_TRY(hip_status(hipEventRecord(g_prof_start, st), where));
    if (shared && gv) {
      MM_TRY(hip_status(mm::launch_gateup_i4_gemv_pair(ar, as, xq, sx, gq, w_gateup.scales, sgq,
                                                       ws_gateup.scales, a_r, a_s, st), where));
    } else if (gu_mfma_pair) {
      MM_TRY(hip_status(mm::launch_gateup_i4_mfma_pair(ar, as, xq, sx, gq, w_gateup.scales, sgq,
                                                       ws_gateup.scales, a_r, a_s, st), where));
    } else {
      MM_TRY(hip_status(gateup_i4(ar, xq, sx, gq, w_gateup.scales, a_r, q_r, s_r, nullptr, st), where));
      if (shared)
        MM_TRY(hip_status(gateup_i4(as, xq, sx, sgq, ws_gateup.scales, a_s, q_s, s_s, nullptr, st),
                          where));
    }
    if (g_prof_stop) MM_TRY(hip_status(hipEventRecord(g_prof_stop, st), where));
    if (quant_pair)
      MM_TRY(hip_status(mm::launch_act_quant_i8_pair(Tk, h, a_r, q_r, s_r, T, hs, a_s, q_s, s_s, st,
                                                     dn_mfma_pair ? mm::kActGroupMajor
                                                                  : mm::kActRowMajor), where));
    // down of both kinds
    if (qin) {
      MM_TRY(hip_status(mm::launch_down_i4_gemv_pair_f32in(ar, as, a_r, a_s, dq, w_down.scales, sdq,
                                                           ws_down.scales, f, ys, st), where));
    } else if (shared && dv) {
      MM_TRY(hip_status(mm::launch_down_i4_gemv_pair(ar, as, q_r, s_r, q_s, s_s, dq, w_down.scales,
                                                     sdq, ws_down.scales, f, ys, st), where));
    } else if (dn_mfma_pair && cmb_in_down) {
      MM_TRY(hip_status(mm::launch_down_i4_mfma_cmb(ar, as, q_r, s_r, q_s, s_s, dq, w_down.scales, sdq,
                                                    ws_down.scales, f, inv, topk_w,
                                                    static_cast<float*>(y), st), where));
      return MM_OK;
    } else if (dn_mfma_pair) {
      MM_TRY(hip_status(mm::launch_down_i4_mfma_pair(ar, as, q_r, s_r, q_s, s_s, dq, w_down.scales,
                                                     sdq, ws_down.scales, f, ys, st), where));
    } else {
      MM_TRY(hip_status(down_i4(ar, q_r, s_r, dq, w_down.scales, f, nullptr, st), where));
      if (shared)
        MM_TRY(hip_status(down_i4(as, q_s, s_s, sdq, ws_down.scales, ys, nullptr, st), where));
    }
  } else if (desc->wfmt == MM_W_BF16) {
    uint16_t* xb = static_cast<uint16_t*>(at(W.xb));
    uint16_t* h_r = static_cast<uint16_t*>(at(W.a_r));
    uint16_t* h_s = static_cast<uint16_t*>(at(W.a_s));
    MM_TRY(hip_status(mm::launch_convert_bf16(T * d, x, xb, st), where));
    if (g_prof_start) MM_TRY(hip_status(hipEventRecord(g_prof_start, st), where));
    MM_TRY(hip_status(mm::launch_gateup_bf16_mfma(ar, xb, static_cast<const uint16_t*>(w_gateup.data),
                                                  h_r, st), where));
    if (shared)
      MM_TRY(hip_status(mm::launch_gateup_bf16_mfma(as, xb, static_cast<const uint16_t*>(ws_gateup.data),
                                                    h_s, st), where));
    if (g_prof_stop) MM_TRY(hip_status(hipEventRecord(g_prof_stop, st), where));
    MM_TRY(hip_status(mm::launch_down_bf16_mfma(ar, h_r, static_cast<const uint16_t*>(w_down.data), f,
                                                st), where));
    if (shared)
      MM_TRY(hip_status(mm::launch_down_bf16_mfma(as, h_s, static_cast<const uint16_t*>(ws_down.data),
                                                  ys, st), where));
  } else {
    void* h_r = at(W.a_r);
    void* h_s = at(W.a_s);
    if (g_prof_start) MM_TRY(hip_status(hipEventRecord(g_prof_start, st), where));
    MM_TRY(hip_status(mm::launch_gateup_fp(ar, false, x, w_gateup.data, h_r, st), where));
    if (shared) MM_TRY(hip_status(mm::launch_gateup_fp(as, false, x, ws_gateup.data, h_s, st), where));
    if (g_prof_stop) MM_TRY(hip_status(hipEventRecord(g_prof_stop, st), where));
    MM_TRY(hip_status(mm::launch_down_fp(ar, false, h_r, w_down.data, f, st), where));
    if (shared) MM_TRY(hip_status(mm::launch_down_fp(as, false, h_s, ws_down.data, ys, st), where));
  }
  return hip_status(mm::launch_combine(T, d, k, f, inv, topk_w, ys, y,
                                       desc->out_dtype == MM_OUT_BF16, st, y_norm, norm_eps),
                    where);
}

int32_t mm_moe_decode_supported(const mm_layer_desc* desc, int64_t T) {
  if (check_desc(desc) != MM_OK) return 0;
  return decode_applies(desc, T) ? 1 : 0;
}

mm_status mm_moe_decode(const mm_layer_desc* desc, int64_t T, const float* x,
                        const float* w_router, const float* bias, mm_weight w_gateup,
                        mm_weight w_down, mm_weight ws_gateup, mm_weight ws_down,
                        int32_t* topk_idx, float* topk_w, void* y, float* y_norm, float norm_eps,
                        void* ws, size_t ws_size, void* stream) {
  auto get_ws = [&](size_t need, char** base) -> mm_status {
    MM_REQUIRE(ws);
    if (ws_size < need)
      return fail(MM_ERR_WORKSPACE, "decode workspace too small (need %lld bytes)", (long long)need);
    *base = static_cast<char*>(ws);
    return MM_OK;
  };
  return moe_decode_impl("mm_moe_decode", desc, T, x, w_router, bias, w_gateup, w_down, ws_gateup,
                         ws_down, topk_idx, topk_w, y, y_norm, norm_eps, stream, get_ws);
}

mm_status mm_moe_decode_noalloc(const mm_layer_desc* desc, int64_t T, const float* x,
                                const float* w_router, const float* bias, mm_weight w_gateup,
                                mm_weight w_down, mm_weight ws_gateup, mm_weight ws_down,
                                int32_t* topk_idx, float* topk_w, void* y, float* y_norm,
                                float norm_eps, void* stream) {
  auto get_ws = [&](size_t need, char** base) -> mm_status {
    if (need > mm::decode_scratch_capacity())
      return fail(MM_ERR_WORKSPACE,
                  "mm_moe_decode_noalloc: the layer needs %lld bytes of scratch, the fixed "
                  "device scratch holds %lld (use mm_moe_decode with a workspace)",
                  (long long)need, (long long)mm::decode_scratch_capacity());
    void* p = nullptr;
    MM_TRY(hip_status(mm::decode_scratch(&p, S(stream)), "mm_moe_decode_noalloc"));
    *base = static_cast<char*>(p);
    return MM_OK;
  };
  return moe_decode_impl("mm_moe_decode_noalloc", desc, T, x, w_router, bias, w_gateup, w_down,
                         ws_gateup, ws_down, topk_idx, topk_w, y, y_norm, norm_eps, stream, get_ws);
}

mm_status mm_linear_w4a8(int64_t rows, int64_t in_features, int64_t out_features,
                         const int8_t* xq, const float* sx, mm_weight w, float* y, void* stream) {
  if (rows < 0) return fail(MM_ERR_SHAPE, "rows %lld is negative", (long long)rows);
  if (in_features < 64 || in_features % 64 || out_features < 64 || out_features % 64)
    return fail(MM_ERR_SHAPE, "in/out features %lld x %lld must be positive multiples of 64",
                (long long)in_features, (long long)out_features);
  if (rows * std::max(in_features, out_features) >= (int64_t(1) << 31))
    return fail(MM_ERR_SHAPE, "rows * features must stay below 2^31");
  if (rows == 0) return MM_OK;
  MM_REQUIRE(xq);
  MM_REQUIRE(sx);
  MM_REQUIRE(w.data);
  MM_REQUIRE(w.scales);
  MM_REQUIRE(y);
  // the dense down-product form: out = a.d = N features from a.h = K inputs
  const mm::ExpertArgs a{rows, rows, (int)out_features, (int)in_features, 1, 1, nullptr, nullptr};
  return hip_status(down_i4(a, xq, sx, static_cast<const uint8_t*>(w.data), w.scales, y, nullptr,
                            S(stream)),
                    "mm_linear_w4a8");
}

static mm_status check_attn(int64_t B, int32_t n_h, int32_t n_kv, int32_t d_h, int64_t max_T) {
  if (B < 0) return fail(MM_ERR_SHAPE, "B %lld is negative", (long long)B);
  if (d_h != 64) return fail(MM_ERR_SHAPE, "d_h %d must be 64", (int)d_h);
  if (n_kv < 1 || n_h < n_kv || n_h % n_kv || n_h / n_kv > 8)
    return fail(MM_ERR_SHAPE, "n_h %d must be a multiple of n_kv %d, at most 8 times it", (int)n_h,
                (int)n_kv);
  if (max_T < 1 || B * n_kv * max_T * d_h >= (int64_t(1) << 40))
    return fail(MM_ERR_SHAPE, "max_T %lld out of range", (long long)max_T);
  return MM_OK;
}

size_t mm_attn_workspace_bytes(int64_t B, int32_t n_kv, int64_t max_len) {
  if (B < 0 || n_kv < 1 || max_len < 1) return 0;
  return std::max<size_t>(mm::attn_partial_bytes(B, n_kv, max_len), 256);
}

mm_status mm_kv_append_i8(int64_t B, int32_t n_kv, int32_t d_h, int64_t max_T, const int32_t* pos,
                          const float* k_new, const float* v_new, int8_t* k_cache,
                          int8_t* v_cache, float* k_scale, float* v_scale, void* stream) {
  MM_TRY(check_attn(B, n_kv, n_kv, d_h, max_T));
  if (B == 0) return MM_OK;
  MM_REQUIRE(pos);
  MM_REQUIRE(k_new);
  MM_REQUIRE(v_new);
  MM_REQUIRE(k_cache);
  MM_REQUIRE(v_cache);
  MM_REQUIRE(k_scale);
  MM_REQUIRE(v_scale);
  return hip_status(mm::launch_kv_append(B, n_kv, max_T, pos, k_new, v_new, k_cache, v_cache,
                                         k_scale, v_scale, S(stream)),
                    "mm_kv_append_i8");
}

mm_status mm_attn_decode_i8(int64_t B, int32_t n_h, int32_t n_kv, int32_t d_h, int64_t max_T,
                            int64_t max_len, const int32_t* lens, const float* q,
                            const int8_t* k_cache, const int8_t* v_cache, const float* k_scale,
                            const float* v_scale, float* out, void* ws, size_t ws_bytes,
                            void* stream) {
  MM_TRY(check_attn(B, n_h, n_kv, d_h, max_T));
  if (max_len < 1 || max_len > max_T)
    return fail(MM_ERR_SHAPE, "max_len %lld must be in [1, max_T]", (long long)max_len);
  if (B == 0) return MM_OK;
  MM_REQUIRE(lens);
  MM_REQUIRE(q);
  MM_REQUIRE(k_cache);
  MM_REQUIRE(v_cache);
  MM_REQUIRE(k_scale);
  MM_REQUIRE(v_scale);
  MM_REQUIRE(out);
  MM_REQUIRE(ws);
  if (ws_bytes < mm::attn_partial_bytes(B, n_kv, max_len))
    return fail(MM_ERR_WORKSPACE, "attention workspace too small (need %zu bytes)",
                mm::attn_partial_bytes(B, n_kv, max_len));
  return hip_status(mm::launch_attn_decode(B, n_h, n_kv, max_T, max_len, lens, q, k_cache, v_cache,
                                           k_scale, v_scale, static_cast<float*>(ws), out,
                                           S(stream)),
                    "mm_attn_decode_i8");
}

mm_status mm_bias_update(int64_t T, int32_t E, int32_t k, const int32_t* topk_idx, float lambda,
                         float* bias, int32_t* load, void* stream) {
  if (T < 0 || E < 1 || E > 4096 || k < 1 || T * k >= (int64_t(1) << 31))
    return fail(MM_ERR_SHAPE, "bias update: T %lld, E %d, k %d out of range", (long long)T, (int)E,
                (int)k);
  if (T == 0) return MM_OK;
  MM_REQUIRE(topk_idx);
  MM_REQUIRE(bias);
  MM_OPTIONAL(load);
  return hip_status(mm::launch_bias_update(T * k, E, topk_idx, lambda, bias, load, S(stream)),
                    "mm_bias_update");
}

int64_t mm_drop_pad_capacity(int64_t T, int32_t k, int32_t E, int32_t num, int32_t den) {
  if (T < 0 || k < 1 || E < 1 || num < 1 || den < 1 || T * k >= (int64_t(1) << 31)) return -1;
  const int64_t a = T * k * num, b = (int64_t)E * den;
  return (a + b - 1) / b;
}

mm_status mm_drop_pad(int64_t T, int32_t E, int32_t k, int64_t capacity, const int32_t* topk_idx,
                      const int32_t* offsets, const int32_t* perm, const int32_t* inv_perm,
                      int32_t* buf, int32_t* offsets_c, int32_t* perm_c, int32_t* inv_c,
                      void* stream) {
  if (T < 0 || E < 1 || E > 4096 || k < 1 || capacity < 0 || T * k >= (int64_t(1) << 31) ||
      (int64_t)E * capacity >= (int64_t(1) << 31))
    return fail(MM_ERR_SHAPE, "drop-and-pad: T %lld, E %d, k %d, capacity %lld out of range",
                (long long)T, (int)E, (int)k, (long long)capacity);
  MM_REQUIRE(offsets);
  MM_REQUIRE(offsets_c);
  if ((int64_t)E * capacity > 0) MM_REQUIRE(buf);
  if (T > 0) {
    MM_REQUIRE(topk_idx);
    MM_REQUIRE(perm);
    MM_REQUIRE(inv_perm);
    MM_REQUIRE(perm_c);
    MM_REQUIRE(inv_c);
  }
  return hip_status(mm::launch_drop_pad(T * k, E, capacity, topk_idx, offsets, perm, inv_perm, buf,
                                        offsets_c, perm_c, inv_c, S(stream)),
                    "mm_drop_pad");
}

mm_status mm_fake_quant(int64_t rows, int64_t cols, int32_t bits, int64_t group, const float* x,
                        float* x_bar, const float* grad_out, float* grad_in, void* stream) {
  if (rows < 0 || cols < 1 || (bits != 4 && bits != 8))
    return fail(MM_ERR_SHAPE, "fake quant: rows %lld, cols %lld, bits %d", (long long)rows,
                (long long)cols, (int)bits);
  const bool row_group = group == cols;
  if (!(group == 32 && cols % 32 == 0) && !(row_group && cols % 4 == 0))
    return fail(MM_ERR_SHAPE, "fake quant: group %lld must be 32 (cols a multiple of 32) or cols "
                "(a multiple of 4)", (long long)group);
  if (rows * cols >= (int64_t(1) << 40)) return fail(MM_ERR_SHAPE, "fake quant: too large");
  if ((grad_out == nullptr) != (grad_in == nullptr))
    return fail(MM_ERR_NULL, "fake quant: grad_out and grad_in must both be set or both NULL");
  if (rows == 0) return MM_OK;
  MM_REQUIRE(x);
  MM_OPTIONAL(x_bar);
  MM_OPTIONAL(grad_out);
  MM_OPTIONAL(grad_in);
  return hip_status(mm::launch_fake_quant(rows, cols, bits, row_group && group != 32, x, x_bar,
                                          grad_out, grad_in, S(stream)),
                    "mm_fake_quant");
}

mm_status mm_gather_rows(int64_t R, int64_t d, int32_t k, const int32_t* perm, const float* scale,
                         const float* src, float* dst, void* stream) {
  if (R < 0 || d < 4 || d % 4 || k < 1 || R * d >= (int64_t(1) << 40))
    return fail(MM_ERR_SHAPE, "gather rows: R %lld, d %lld, k %d", (long long)R, (long long)d, (int)k);
  if (R == 0) return MM_OK;
  MM_REQUIRE(perm);
  MM_OPTIONAL(scale);
  MM_REQUIRE(src);
  MM_REQUIRE(dst);
  return hip_status(mm::launch_gather_rows(R, d, k, perm, scale, src, dst, S(stream)),
                    "mm_gather_rows");
}

static mm_status check_train(int32_t E, int32_t d, int32_t h, int64_t R) {
  if (E < 1 || E > 4096 || d < 16 || d % 16 || h < 16 || h % 16 || R < 0 ||
      R >= (int64_t(1) << 31) || R * 2 * h >= (int64_t(1) << 40) || R * d >= (int64_t(1) << 40))
    return fail(MM_ERR_SHAPE, "expert training pass: E %d, d %d, h %d, R %lld (d, h multiples of 16)",
                (int)E, (int)d, (int)h, (long long)R);
  return MM_OK;
}

mm_status mm_expert_train_forward_f32(int32_t E, int32_t d, int32_t h, int64_t R,
                                      const int32_t* offsets, const float* xs, const float* w_gu,
                                      const float* w_d, float* gu, float* a_bar, float* f,
                                      void* stream) {
  MM_TRY(check_train(E, d, h, R));
  if (R == 0) return MM_OK;
  MM_REQUIRE(offsets);
  MM_REQUIRE(xs);
  MM_REQUIRE(w_gu);
  MM_REQUIRE(w_d);
  MM_REQUIRE(gu);
  MM_REQUIRE(a_bar);
  MM_REQUIRE(f);
  return hip_status(mm::launch_expert_train_forward(E, d, h, R, offsets, xs, w_gu, w_d, gu, a_bar, f,
                                                    S(stream)),
                    "mm_expert_train_forward_f32");
}

size_t mm_expert_backward_workspace_bytes(int64_t R, int32_t h) {
  if (R < 0 || h < 1) return 0;
  return std::max<size_t>((size_t)R * 3 * h * sizeof(float), 256);
}

mm_status mm_expert_backward_f32(int32_t E, int32_t d, int32_t h, int64_t R, const int32_t* offsets,
                                 const float* xs, const float* w_gu, const float* w_d,
                                 const float* gu, const float* a_bar, const float* df, float* dxs,
                                 float* dw_gu, float* dw_d, void* ws, size_t ws_bytes,
                                 void* stream) {
  MM_TRY(check_train(E, d, h, R));
  MM_REQUIRE(offsets);
  MM_REQUIRE(w_gu);
  MM_REQUIRE(w_d);
  MM_REQUIRE(dw_gu);
  MM_REQUIRE(dw_d);
  if (R > 0) {
    MM_REQUIRE(xs);
    MM_REQUIRE(gu);
    MM_REQUIRE(a_bar);
    MM_REQUIRE(df);
    MM_REQUIRE(dxs);
    MM_REQUIRE(ws);
    if (ws_bytes < (size_t)R * 3 * h * sizeof(float))
      return fail(MM_ERR_WORKSPACE, "expert backward workspace too small (need %zu bytes)",
                  (size_t)R * 3 * h * sizeof(float));
  }
  float* dabar = static_cast<float*>(ws);
  float* dgu = dabar + R * h;
  return hip_status(mm::launch_expert_backward(E, d, h, R, offsets, xs, w_gu, w_d, gu, a_bar, df,
                                               dxs, dw_gu, dw_d, dabar, dgu, S(stream)),
                    "mm_expert_backward_f32");
}

mm_status mm_router_backward_f32(const mm_layer_desc* desc, int64_t T, const float* x,
                                 const float* w_router, const float* bias, const int32_t* topk_idx,
                                 const float* f, const int32_t* inv, const float* dy,
                                 float lambda_z, float* dz, float* dw_router, float* dx,
                                 void* stream) {
  MM_REQUIRE(desc);
  const int E = desc->n_experts, d = desc->d_model, k = desc->top_k;
  if (T < 1 || E < 4 || E > 64 || E % 4 || d < 16 || d % 16 || k < 1 || k > E ||
      desc->gating < 0 || desc->gating > 3 || T * (int64_t)d >= (int64_t(1) << 40))
    return fail(MM_ERR_SHAPE, "router backward: T %lld, E %d (<= 64, multiple of 4), d %d "
                "(multiple of 16), k %d", (long long)T, E, d, k);
  MM_REQUIRE(x);
  MM_REQUIRE(w_router);
  MM_OPTIONAL(bias);
  MM_REQUIRE(topk_idx);
  MM_REQUIRE(f);
  MM_REQUIRE(inv);
  MM_REQUIRE(dy);
  MM_REQUIRE(dz);
  MM_REQUIRE(dw_router);
  MM_REQUIRE(dx);
  return hip_status(mm::launch_router_backward(T, d, E, k, desc->gating, x, w_router, bias, topk_idx,
                                               f, inv, dy, lambda_z, dz, dw_router, dx, S(stream)),
                    "mm_router_backward_f32");
}

mm_status mm_rmsnorm_f32(int64_t rows, int64_t cols, float eps, const float* x, float* y,
                         void* stream) {
  if (rows < 0 || cols <= 0) return fail(MM_ERR_SHAPE, "bad shape");
  if (rows == 0) return MM_OK;
  MM_REQUIRE(x);
  MM_REQUIRE(y);
  return hip_status(mm::launch_rmsnorm(rows, cols, eps, x, y, S(stream)), "mm_rmsnorm_f32");
}

mm_status mm_add_rmsnorm_f32(int64_t rows, int64_t cols, float eps, const float* x, const float* r,
                             float* sum, float* norm, void* stream) {
  if (rows < 0 || cols <= 0) return fail(MM_ERR_SHAPE, "bad shape");
  if (norm && !(eps > 0.0f)) return fail(MM_ERR_SHAPE, "eps must be positive");
  if (rows == 0) return MM_OK;
  MM_REQUIRE(x);
  MM_REQUIRE(r);
  MM_REQUIRE(sum);
  MM_OPTIONAL(norm);
  if (sum == x || sum == r || (norm && (norm == x || norm == r || norm == sum)))
    return fail(MM_ERR_SHAPE, "outputs must not alias the inputs or each other");
  return hip_status(mm::launch_add_rmsnorm(rows, cols, eps, x, r, sum, norm, S(stream)),
                    "mm_add_rmsnorm_f32");
}

size_t mm_kv_cache_bytes(int64_t B, int32_t n_kv, int32_t d_h, int64_t max_T, int32_t which) {
  if (B < 0 || n_kv < 1 || d_h < 1 || max_T < 0) return 0;
  const size_t vectors = (size_t)B * (size_t)n_kv * (size_t)max_T;
  switch (which) {
    case MM_KV_CODES: return vectors * (size_t)d_h;  // one byte per value
    case MM_KV_SCALES: return vectors * sizeof(float);
    default: return 0;
  }
}

}  // extern "C"
