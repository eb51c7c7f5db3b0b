// libncattn C ABI: argument validation and dispatch. Every entry point
// checks its arguments before any HIP call, then checks that the current
// device is a gfx950, enqueues its kernels on the caller's stream and
// returns without synchronising.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/ncattn.h"
#include "kernels.hpp"

namespace nc {
bool decode_group_supported(int G);
}

namespace {

thread_local char g_msg[512] = "";
thread_local nc::BwdEvents g_bwd_ev = {nullptr, nullptr, nullptr};
thread_local hipEvent_t g_fwd_ev[3] = {nullptr, nullptr, nullptr};  // k prologue, forward, end

nc_status fail(nc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return s;
}

constexpr long long kMaxElems = 2147483647LL;  // per-tensor element count limit (int32 indexing margin)
constexpr int kMaxGridYZ = 65535;              // largest second / third grid dimension

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Common shape checks of the attention entry points.
nc_status check_shape(nc_dtype dt, int B, int T, int H, int Hkv, int D) {
  if (dt != NC_F32 && dt != NC_BF16) return fail(NC_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (B < 1 || T < 1 || H < 1 || Hkv < 1 || D < 1)
    return fail(NC_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d T=%d H=%d Hkv=%d D=%d)", B, T, H, Hkv, D);
  if (H % Hkv != 0) return fail(NC_ERR_INVALID_ARG, "H=%d is not a multiple of Hkv=%d", H, Hkv);
  if (D != 32 && D != 64 && D != 128) return fail(NC_ERR_UNSUPPORTED, "head dim D=%d not in {32, 64, 128}", D);
  if ((long long)B * T * H * D > kMaxElems)
    return fail(NC_ERR_UNSUPPORTED, "tensor of B*T*H*D=%lld elements exceeds 2^31-1", (long long)B * T * H * D);
  // the float32 kernels put heads and rows on the second and third grid axes
  if (dt == NC_F32 && (B > kMaxGridYZ || H > kMaxGridYZ))
    return fail(NC_ERR_UNSUPPORTED, "float32 path: B=%d and H=%d must be <= %d", B, H, kMaxGridYZ);
  return NC_OK;
}

// Decode grids: rows on the third axis, chunks of the cache on the second.
nc_status check_decode_grid(int B, int T_max, int D, int G) {
  if (B > kMaxGridYZ) return fail(NC_ERR_UNSUPPORTED, "decode: B=%d exceeds %d rows", B, kMaxGridYZ);
  const int chunk = nc::decode_chunk(D, G);
  if ((T_max + chunk - 1) / chunk > kMaxGridYZ)
    return fail(NC_ERR_UNSUPPORTED, "decode: T_max=%d exceeds %lld positions at D=%d", T_max,
                (long long)kMaxGridYZ * chunk, D);
  return NC_OK;
}

nc_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(NC_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(NC_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return NC_OK;
}

nc_status check_scale(float scale) {
  if (!(scale > 0.f) || !isfinite(scale)) return fail(NC_ERR_INVALID_ARG, "scale must be finite and > 0");
  return NC_OK;
}

// The current device must be a gfx950. Properties are cached per device id.
nc_status check_device(int* dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(NC_ERR_DEVICE, "no HIP device available");
  }
  static std::mutex mu;
  static int known[64];  // 0 unknown, 1 gfx950, 2 other
  if (dev >= 64) return fail(NC_ERR_DEVICE, "device id %d out of range", dev);
  int state;
  {
    std::lock_guard<std::mutex> lk(mu);
    state = known[dev];
  }
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(NC_ERR_DEVICE, "cannot query device %d", dev);
    }
    state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    std::lock_guard<std::mutex> lk(mu);
    known[dev] = state;
  }
  if (state != 1) return fail(NC_ERR_DEVICE, "device %d is not a gfx950", dev);
  if (dev_out) *dev_out = dev;
  return NC_OK;
}

nc_status finish(hipError_t e, hipStream_t s, const char* what) {
  if (e != hipSuccess) return fail(NC_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  static const bool debug_sync = getenv("NC_DEBUG_SYNC") && getenv("NC_DEBUG_SYNC")[0] == '1';
  if (debug_sync) {
    e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(NC_ERR_LAUNCH, "%s: kernel failed: %s", what, hipGetErrorString(e));
  }
  g_msg[0] = 0;
  return NC_OK;
}

#define NC_TRY(x)                \
  do {                           \
    nc_status _st = (x);         \
    if (_st != NC_OK) return _st; \
  } while (0)

int norm_window(int window, int T) { return (window <= 0 || window >= T) ? 0 : window; }

int decode_splits(int T_max, int D, int G) {
  const int chunk = nc::decode_chunk(D, G);
  return (T_max + chunk - 1) / chunk;
}

}  // namespace

extern "C" {

int nc_abi_version(void) { return NCATTN_ABI_VERSION; }

const char* nc_status_string(nc_status s) {
  switch (s) {
    case NC_OK: return "ok";
    case NC_ERR_INVALID_ARG: return "invalid argument";
    case NC_ERR_UNSUPPORTED: return "unsupported";
    case NC_ERR_WORKSPACE: return "workspace too small";
    case NC_ERR_DEVICE: return "no usable gfx950 device";
    case NC_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* nc_last_error_message(void) { return g_msg; }

nc_status nc_attn_fwd(nc_dtype dt, int B, int T, int H, int Hkv, int D, const void* q, const void* k,
                      const void* v, int window, float scale, void* out, float* lse, nc_stream stream) {
  NC_TRY(check_shape(dt, B, T, H, Hkv, D));
  NC_TRY(check_ptr(q, "q"));
  NC_TRY(check_ptr(k, "k"));
  NC_TRY(check_ptr(v, "v"));
  NC_TRY(check_ptr(out, "out"));
  NC_TRY(check_ptr(lse, "lse"));
  NC_TRY(check_scale(scale));
  NC_TRY(check_device(nullptr));
  nc::FwdParams p{q, k, v, out, lse, B, T, H, Hkv, D, norm_window(window, T), scale, scale * 1.4426950408889634f,
                  nullptr, T, nullptr, nullptr, nullptr, nullptr, 0, 0.f};
  hipStream_t s = (hipStream_t)stream;
  return finish(dt == NC_BF16 ? nc::launch_attn_fwd_bf16(p, s) : nc::launch_attn_fwd_f32(p, s), s, "nc_attn_fwd");
}

nc_status nc_attn_fwd_fp8(int B, int T, int H, int Hkv, int D, const void* q, const void* k, const void* v,
                          float q_descale, float k_descale, float v_descale, int window, float scale, void* out,
                          float* lse, nc_stream stream) {
  NC_TRY(check_shape(NC_BF16, B, T, H, Hkv, D));
  if (D != 64 && D != 128) return fail(NC_ERR_UNSUPPORTED, "fp8 forward: head dim D=%d not in {64, 128}", D);
  NC_TRY(check_ptr(q, "q"));
  NC_TRY(check_ptr(k, "k"));
  NC_TRY(check_ptr(v, "v"));
  NC_TRY(check_ptr(out, "out"));
  NC_TRY(check_ptr(lse, "lse"));
  NC_TRY(check_scale(scale));
  const float ds[3] = {q_descale, k_descale, v_descale};
  for (float d : ds)
    if (!(d > 0.f) || !isfinite(d)) return fail(NC_ERR_INVALID_ARG, "descales must be finite and > 0");
  const double sl2 = (double)scale * q_descale * k_descale * 1.4426950408889634;
  if (!(sl2 > 0.0) || !isfinite((float)sl2))
    return fail(NC_ERR_INVALID_ARG, "scale * q_descale * k_descale is not a finite float");
  NC_TRY(check_device(nullptr));
  nc::Fp8FwdParams p{q, k, v, out, lse, B, T, H, Hkv, D, norm_window(window, T), (float)sl2, v_descale};
  hipStream_t s = (hipStream_t)stream;
  return finish(nc::launch_attn_fwd_fp8(p, s), s, "nc_attn_fwd_fp8");
}

nc_status nc_attn_fwd_cache(nc_dtype dt, int B, int Tq, int H, int Hkv, int D, int T_max, const void* q,
                            const void* k_cache, const void* v_cache, const int32_t* cache_seqlens, int window,
                            float scale, void* out, float* lse, nc_stream stream) {
  NC_TRY(check_shape(dt, B, Tq, H, Hkv, D));
  if (T_max < Tq) return fail(NC_ERR_INVALID_ARG, "T_max=%d is smaller than the chunk Tq=%d", T_max, Tq);
  if ((long long)B * T_max * Hkv * D > kMaxElems)
    return fail(NC_ERR_UNSUPPORTED, "cache of B*T_max*Hkv*D elements exceeds 2^31-1");
  NC_TRY(check_ptr(q, "q"));
  NC_TRY(check_ptr(k_cache, "k_cache"));
  NC_TRY(check_ptr(v_cache, "v_cache"));
  if (!cache_seqlens) return fail(NC_ERR_INVALID_ARG, "cache_seqlens is NULL");
  if (((uintptr_t)cache_seqlens & 3u) != 0) return fail(NC_ERR_INVALID_ARG, "cache_seqlens is not 4-byte aligned");
  NC_TRY(check_ptr(out, "out"));
  NC_TRY(check_ptr(lse, "lse"));
  NC_TRY(check_scale(scale));
  NC_TRY(check_device(nullptr));
  nc::FwdParams p{q, k_cache, v_cache, out, lse, B, Tq, H, Hkv, D, norm_window(window, T_max), scale,
                  scale * 1.4426950408889634f, cache_seqlens, T_max, nullptr, nullptr, nullptr, nullptr, 0, 0.f};
  hipStream_t s = (hipStream_t)stream;
  return finish(dt == NC_BF16 ? nc::launch_attn_fwd_bf16(p, s) : nc::launch_attn_fwd_f32(p, s), s,
                "nc_attn_fwd_cache");
}

nc_status nc_kv_cache_append(nc_dtype dt, int B, int Tq, int Hkv, int D, int T_max, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache, const int32_t* cache_seqlens,
                             nc_stream stream) {
  NC_TRY(check_shape(dt, B, Tq, Hkv, Hkv, D));
  if (T_max < Tq) return fail(NC_ERR_INVALID_ARG, "T_max=%d is smaller than the chunk Tq=%d", T_max, Tq);
  if ((long long)B * T_max * Hkv * D > kMaxElems)
    return fail(NC_ERR_UNSUPPORTED, "cache of B*T_max*Hkv*D elements exceeds 2^31-1");
  NC_TRY(check_ptr(k_new, "k_new"));
  NC_TRY(check_ptr(v_new, "v_new"));
  NC_TRY(check_ptr(k_cache, "k_cache"));
  NC_TRY(check_ptr(v_cache, "v_cache"));
  if (!cache_seqlens) return fail(NC_ERR_INVALID_ARG, "cache_seqlens is NULL");
  if (((uintptr_t)cache_seqlens & 3u) != 0) return fail(NC_ERR_INVALID_ARG, "cache_seqlens is not 4-byte aligned");
  NC_TRY(check_device(nullptr));
  hipStream_t s = (hipStream_t)stream;
  return finish(nc::launch_cache_append(k_new, v_new, k_cache, v_cache, cache_seqlens, B, Tq, Hkv, D, T_max,
                                        dt == NC_BF16 ? 2 : 4, s),
                s, "nc_kv_cache_append");
}

size_t nc_attn_bwd_workspace_bytes(nc_dtype dt, int B, int T, int H, int Hkv, int D) {
  if (check_shape(dt, B, T, H, Hkv, D) != NC_OK) return 0;
  size_t row_stats = (size_t)B * H * T * 4;  // delta, then lse * log2(e)
  row_stats = (row_stats + 255) & ~(size_t)255;
  return 2 * row_stats;
}

nc_status nc_attn_bwd(nc_dtype dt, int B, int T, int H, int Hkv, int D, const void* q, const void* k,
                      const void* v, const void* out, const float* lse, const void* dout, int window,
                      float scale, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      nc_stream stream) {
  NC_TRY(check_shape(dt, B, T, H, Hkv, D));
  NC_TRY(check_ptr(q, "q"));
  NC_TRY(check_ptr(k, "k"));
  NC_TRY(check_ptr(v, "v"));
  NC_TRY(check_ptr(out, "out"));
  NC_TRY(check_ptr(lse, "lse"));
  NC_TRY(check_ptr(dout, "dout"));
  NC_TRY(check_ptr(dq, "dq"));
  NC_TRY(check_ptr(dk, "dk"));
  NC_TRY(check_ptr(dv, "dv"));
  NC_TRY(check_scale(scale));
  const size_t need = nc_attn_bwd_workspace_bytes(dt, B, T, H, Hkv, D);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need)
    return fail(NC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  NC_TRY(check_device(nullptr));
  const size_t stat_bytes = ((size_t)B * H * T * 4 + 255) & ~(size_t)255;
  nc::BwdParams p{q, k, v, out, lse, dout, dq, dk, dv, (float*)workspace,
                  (float*)((char*)workspace + stat_bytes),
                  B, T, H, Hkv, D, norm_window(window, T), scale, scale * 1.4426950408889634f,
                  nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0.f};
  hipStream_t s = (hipStream_t)stream;
  return finish(dt == NC_BF16 ? nc::launch_attn_bwd_bf16(p, s, g_bwd_ev) : nc::launch_attn_bwd_f32(p, s, g_bwd_ev),
                s, "nc_attn_bwd");
}

static nc_status prologue_common(nc_dtype dt, int B, int T, int H, int Hkv, int D, const void* q, const void* k,
                                 const int32_t* pos_offset, const float* cos_tab, const float* sin_tab,
                                 int T_rope, float eps);

nc_status nc_attn_bwd_prologue(nc_dtype dt, int B, int T, int H, int Hkv, int D, const void* q, const void* k,
                               const void* v, const void* out, const float* lse, const void* dout, int window,
                               float scale, const void* q_raw, const void* k_raw, const int32_t* pos_offset,
                               const float* cos_tab, const float* sin_tab, int T_rope, float eps, void* dq,
                               void* dk, void* dv, void* workspace, size_t workspace_bytes, nc_stream stream) {
  NC_TRY(check_shape(dt, B, T, H, Hkv, D));
  NC_TRY(check_ptr(q, "q"));
  NC_TRY(check_ptr(k, "k"));
  NC_TRY(check_ptr(v, "v"));
  NC_TRY(check_ptr(out, "out"));
  NC_TRY(check_ptr(lse, "lse"));
  NC_TRY(check_ptr(dout, "dout"));
  NC_TRY(check_ptr(dq, "dq"));
  NC_TRY(check_ptr(dk, "dk"));
  NC_TRY(check_ptr(dv, "dv"));
  NC_TRY(check_scale(scale));
  NC_TRY(prologue_common(dt, B, T, H, Hkv, D, q_raw, k_raw, pos_offset, cos_tab, sin_tab, T_rope, eps));
  const size_t need = nc_attn_bwd_workspace_bytes(dt, B, T, H, Hkv, D);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need)
    return fail(NC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  NC_TRY(check_device(nullptr));
  const size_t stat_bytes = ((size_t)B * H * T * 4 + 255) & ~(size_t)255;
  const bool bf16 = dt == NC_BF16;
  // bf16: the two backward kernels apply the prologue backward before storing dq, dk.
  // float32: attention gradients into dq, dk, then the prologue backward in place
  // (each head vector is read whole before it is written).
  nc::BwdParams p{q, k, v, out, lse, dout, dq, dk, dv, (float*)workspace,
                  (float*)((char*)workspace + stat_bytes),
                  B, T, H, Hkv, D, norm_window(window, T), scale, scale * 1.4426950408889634f,
                  bf16 ? q_raw : nullptr, bf16 ? k_raw : nullptr, pos_offset, cos_tab, sin_tab, T_rope, eps};
  hipStream_t s = (hipStream_t)stream;
  if (bf16) return finish(nc::launch_attn_bwd_bf16(p, s, g_bwd_ev), s, "nc_attn_bwd_prologue");
  hipError_t e = nc::launch_attn_bwd_f32(p, s, g_bwd_ev);
  if (e == hipSuccess) {
    nc::PrologueParams pp{q_raw, k_raw, pos_offset, cos_tab, sin_tab, dq, dk, dq, dk, B, T, H, Hkv, D, T_rope, eps};
    e = nc::launch_prologue(pp, false, true, s);
  }
  return finish(e, s, "nc_attn_bwd_prologue");
}

nc_status nc_profile_bwd_main(void* dq_begin, void* dkdv_begin, void* end) {
  const int set = (dq_begin != nullptr) + (dkdv_begin != nullptr) + (end != nullptr);
  if (set != 0 && set != 3) return fail(NC_ERR_INVALID_ARG, "the three events must all be set or all be NULL");
  g_bwd_ev = {(hipEvent_t)dq_begin, (hipEvent_t)dkdv_begin, (hipEvent_t)end};
  g_msg[0] = 0;
  return NC_OK;
}

size_t nc_attn_decode_workspace_bytes(nc_dtype dt, int B, int H, int Hkv, int D, int T_max) {
  if (check_shape(dt, B, T_max, H, Hkv, D) != NC_OK) return 0;
  return (size_t)B * H * decode_splits(T_max, D, H / Hkv) * (D + 2) * 4;
}

nc_status nc_attn_decode(nc_dtype dt, int B, int H, int Hkv, int D, int T_max, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* seqlens, int window,
                         float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                         nc_stream stream) {
  NC_TRY(check_shape(dt, B, T_max, H, Hkv, D));
  if ((long long)B * T_max * Hkv * D > kMaxElems)
    return fail(NC_ERR_UNSUPPORTED, "cache of B*T_max*Hkv*D elements exceeds 2^31-1");
  if (!nc::decode_group_supported(H / Hkv))
    return fail(NC_ERR_UNSUPPORTED, "decode supports query groups H/Hkv in {1,2,3,4,6,8}, got %d", H / Hkv);
  NC_TRY(check_decode_grid(B, T_max, D, H / Hkv));
  NC_TRY(check_ptr(q, "q"));
  NC_TRY(check_ptr(k_cache, "k_cache"));
  NC_TRY(check_ptr(v_cache, "v_cache"));
  if (!seqlens) return fail(NC_ERR_INVALID_ARG, "seqlens is NULL");
  if (((uintptr_t)seqlens & 3u) != 0) return fail(NC_ERR_INVALID_ARG, "seqlens is not 4-byte aligned");
  NC_TRY(check_ptr(out, "out"));
  if (!lse) return fail(NC_ERR_INVALID_ARG, "lse is NULL");
  if (((uintptr_t)lse & 3u) != 0) return fail(NC_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  NC_TRY(check_scale(scale));
  const size_t need = nc_attn_decode_workspace_bytes(dt, B, H, Hkv, D, T_max);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need)
    return fail(NC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  NC_TRY(check_device(nullptr));
  nc::DecodeParams p{q, k_cache, v_cache, seqlens, out, lse, (float*)workspace, B, H, Hkv, D, T_max,
                     window <= 0 ? 0 : window, decode_splits(T_max, D, H / Hkv), scale,
                     scale * 1.4426950408889634f};
  hipStream_t s = (hipStream_t)stream;
  return finish(nc::launch_decode(p, dt == NC_BF16, s), s, "nc_attn_decode");
}


size_t nc_attn_decode_step_workspace_bytes(nc_dtype dt, int B, int H, int Hkv, int D, int T_max) {
  return nc_attn_decode_workspace_bytes(dt, B, H, Hkv, D, T_max);  // the split-K partials only
}

namespace {

// Validation shared by the two decode-step entry points (everything but the
// workspace).
nc_status decode_step_checks(nc_dtype dt, int B, int H, int Hkv, int D, int T_max, const void* q,
                             const void* k_new, const void* v_new, const void* k_cache, const void* v_cache,
                             const int32_t* cache_seqlens, const float* cos_tab, const float* sin_tab, int T_rope,
                             float eps, float scale, const void* out, const float* lse) {
  NC_TRY(check_shape(dt, B, T_max, H, Hkv, D));
  if ((long long)B * T_max * Hkv * D > kMaxElems)
    return fail(NC_ERR_UNSUPPORTED, "cache of B*T_max*Hkv*D elements exceeds 2^31-1");
  if (!nc::decode_group_supported(H / Hkv))
    return fail(NC_ERR_UNSUPPORTED, "decode supports query groups H/Hkv in {1,2,3,4,6,8}, got %d", H / Hkv);
  NC_TRY(check_decode_grid(B, T_max, D, H / Hkv));
  NC_TRY(check_ptr(q, "q"));
  NC_TRY(check_ptr(k_new, "k_new"));
  NC_TRY(check_ptr(v_new, "v_new"));
  NC_TRY(check_ptr(k_cache, "k_cache"));
  NC_TRY(check_ptr(v_cache, "v_cache"));
  if (!cache_seqlens) return fail(NC_ERR_INVALID_ARG, "cache_seqlens is NULL");
  if (((uintptr_t)cache_seqlens & 3u) != 0) return fail(NC_ERR_INVALID_ARG, "cache_seqlens is not 4-byte aligned");
  NC_TRY(check_ptr(cos_tab, "cos"));
  NC_TRY(check_ptr(sin_tab, "sin"));
  if (T_rope < 1) return fail(NC_ERR_INVALID_ARG, "T_rope must be >= 1");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(NC_ERR_INVALID_ARG, "eps must be finite and >= 0");
  NC_TRY(check_ptr(out, "out"));
  if (!lse) return fail(NC_ERR_INVALID_ARG, "lse is NULL");
  if (((uintptr_t)lse & 3u) != 0) return fail(NC_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  NC_TRY(check_scale(scale));
  return NC_OK;
}

nc_status decode_step_launch(nc_dtype dt, int B, int H, int Hkv, int D, int T_max, const void* q, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache, const int32_t* cache_seqlens,
                             const float* cos_tab, const float* sin_tab, int T_rope, float eps, int window,
                             float scale, void* out, float* lse, float* part, nc_stream stream, const char* what) {
  // the split kernel applies the prologue and writes the cache slot itself
  nc::DecodeParams p{q, k_cache, v_cache, cache_seqlens, out, lse, part, B, H, Hkv, D, T_max,
                     window <= 0 ? 0 : window, decode_splits(T_max, D, H / Hkv), scale,
                     scale * 1.4426950408889634f, 1, k_new, v_new, cos_tab, sin_tab, T_rope, eps};
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = nc::launch_decode(p, dt == NC_BF16, s);
  return finish(e, s, what);
}

// Scratch of the entry point that allocates nothing: a file-scope device
// array, one copy per GPU (the runtime places it when it loads this code
// object on a device and keeps it until the process ends). In host code the
// array's name is only a stand-in for the symbol; its device address differs
// per GPU and comes from hipGetSymbolAddress, taken once per device with that
// device current and cached here. Every use passes that address.
static __device__ __align__(256) unsigned char scratch[NC_NOALLOC_SCRATCH_BYTES];

nc_status scratch_ptr(int dev, void** out) {
  static std::mutex mu;
  static void* ptrs[64];
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(NC_ERR_DEVICE, "scratch: hipGetSymbolAddress failed on device %d: %s", dev, hipGetErrorString(e));
    }
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return NC_OK;
}

}  // namespace

nc_status nc_attn_decode_step(nc_dtype dt, int B, int H, int Hkv, int D, int T_max, const void* q,
                              const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* cache_seqlens, const float* cos_tab, const float* sin_tab, int T_rope,
                              float eps, int window, float scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, nc_stream stream) {
  NC_TRY(decode_step_checks(dt, B, H, Hkv, D, T_max, q, k_new, v_new, k_cache, v_cache, cache_seqlens, cos_tab,
                            sin_tab, T_rope, eps, scale, out, lse));
  const size_t need = nc_attn_decode_step_workspace_bytes(dt, B, H, Hkv, D, T_max);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need)
    return fail(NC_ERR_WORKSPACE, "workspace needs %zu bytes (16-byte aligned), got %zu", need, workspace_bytes);
  NC_TRY(check_device(nullptr));
  return decode_step_launch(dt, B, H, Hkv, D, T_max, q, k_new, v_new, k_cache, v_cache, cache_seqlens, cos_tab,
                            sin_tab, T_rope, eps, window, scale, out, lse, (float*)workspace, stream,
                            "nc_attn_decode_step");
}

nc_status nc_attn_decode_step_noalloc(nc_dtype dt, int B, int H, int Hkv, int D, int T_max, const void* q,
                                      const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                      const int32_t* cache_seqlens, const float* cos_tab, const float* sin_tab,
                                      int T_rope, float eps, int window, float scale, void* out, float* lse,
                                      nc_stream stream) {
  NC_TRY(decode_step_checks(dt, B, H, Hkv, D, T_max, q, k_new, v_new, k_cache, v_cache, cache_seqlens, cos_tab,
                            sin_tab, T_rope, eps, scale, out, lse));
  const size_t need = nc_attn_decode_step_workspace_bytes(dt, B, H, Hkv, D, T_max);
  if (need > (size_t)NC_NOALLOC_SCRATCH_BYTES)
    return fail(NC_ERR_UNSUPPORTED, "these sizes need %zu bytes of scratch; the library's scratch holds %zu",
                need, (size_t)NC_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  NC_TRY(check_device(&dev));
  void* part = nullptr;
  NC_TRY(scratch_ptr(dev, &part));
  return decode_step_launch(dt, B, H, Hkv, D, T_max, q, k_new, v_new, k_cache, v_cache, cache_seqlens, cos_tab,
                            sin_tab, T_rope, eps, window, scale, out, lse, (float*)part, stream,
                            "nc_attn_decode_step_noalloc");
}

nc_status nc_kv_cache_replicate(nc_dtype dt, int n_rows, int T_max, int Hkv, int D, int n_tokens, const void* src,
                                void* dst, nc_stream stream) {
  NC_TRY(check_shape(dt, n_rows, T_max, Hkv, Hkv, D));
  if ((long long)n_rows * T_max * Hkv * D > kMaxElems)
    return fail(NC_ERR_UNSUPPORTED, "cache of n_rows*T_max*Hkv*D elements exceeds 2^31-1");
  if (n_tokens < 1 || n_tokens > T_max)
    return fail(NC_ERR_INVALID_ARG, "n_tokens=%d must lie in 1..T_max=%d", n_tokens, T_max);
  NC_TRY(check_ptr(src, "src"));
  NC_TRY(check_ptr(dst, "dst"));
  NC_TRY(check_device(nullptr));
  const size_t es = dt == NC_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)Hkv * D * es;  // one cache position, a multiple of 16 bytes
  hipStream_t s = (hipStream_t)stream;
  return finish(nc::launch_replicate(src, dst, (size_t)n_tokens * row_bytes, n_rows, (size_t)T_max * row_bytes, s),
                s, "nc_kv_cache_replicate");
}

nc_status nc_rope_table(int T_rope, int D, double base, float* cos_out, float* sin_out, nc_stream stream) {
  if (T_rope < 1) return fail(NC_ERR_INVALID_ARG, "T_rope must be >= 1");
  if (D < 2 || D > 256 || (D & 1)) return fail(NC_ERR_INVALID_ARG, "D must be even, 2..256");
  if (!(base > 1.0) || !isfinite(base)) return fail(NC_ERR_INVALID_ARG, "base must be finite and > 1");
  if ((long long)T_rope * (D / 2) > kMaxElems) return fail(NC_ERR_UNSUPPORTED, "table too large");
  if (!cos_out || !sin_out) return fail(NC_ERR_INVALID_ARG, "table pointer is NULL");
  if (((uintptr_t)cos_out & 3u) || ((uintptr_t)sin_out & 3u))
    return fail(NC_ERR_INVALID_ARG, "table pointers must be 4-byte aligned");
  NC_TRY(check_device(nullptr));
  hipStream_t s = (hipStream_t)stream;
  return finish(nc::launch_rope_table(T_rope, D, base, cos_out, sin_out, s), s, "nc_rope_table");
}

static nc_status prologue_common(nc_dtype dt, int B, int T, int H, int Hkv, int D, const void* q, const void* k,
                                 const int32_t* pos_offset, const float* cos_tab, const float* sin_tab,
                                 int T_rope, float eps) {
  NC_TRY(check_shape(dt, B, T, H, Hkv, D));
  NC_TRY(check_ptr(q, "q"));
  NC_TRY(check_ptr(k, "k"));
  NC_TRY(check_ptr(cos_tab, "cos"));
  NC_TRY(check_ptr(sin_tab, "sin"));
  if (pos_offset && ((uintptr_t)pos_offset & 3u)) return fail(NC_ERR_INVALID_ARG, "pos_offset is not 4-byte aligned");
  if (T_rope < 1) return fail(NC_ERR_INVALID_ARG, "T_rope must be >= 1");
  if (!pos_offset && T > T_rope) return fail(NC_ERR_INVALID_ARG, "T=%d exceeds the table length %d", T, T_rope);
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(NC_ERR_INVALID_ARG, "eps must be finite and >= 0");
  return NC_OK;
}

nc_status nc_attn_fwd_prologue(nc_dtype dt, int B, int T, int H, int Hkv, int D, const void* q_raw,
                               const void* k_raw, const void* v, const int32_t* pos_offset, const float* cos_tab,
                               const float* sin_tab, int T_rope, float eps, int window, float scale, void* q_out,
                               void* k_out, void* out, float* lse, nc_stream stream) {
  NC_TRY(prologue_common(dt, B, T, H, Hkv, D, q_raw, k_raw, pos_offset, cos_tab, sin_tab, T_rope, eps));
  NC_TRY(check_ptr(v, "v"));
  NC_TRY(check_ptr(q_out, "q_out"));
  NC_TRY(check_ptr(k_out, "k_out"));
  NC_TRY(check_ptr(out, "out"));
  NC_TRY(check_ptr(lse, "lse"));
  NC_TRY(check_scale(scale));
  NC_TRY(check_device(nullptr));
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dt == NC_BF16;
  // bf16: the keys' prologue alone (no query rows), then the forward applies
  // the queries' prologue as it loads them. float32: both prologues, then the
  // plain forward on their outputs.
  nc::PrologueParams pp{q_raw, k_raw, pos_offset, cos_tab, sin_tab, nullptr, nullptr, q_out, k_out,
                        B, T, bf16 ? 0 : H, Hkv, D, T_rope, eps};
  hipError_t e = hipSuccess;
  if (g_fwd_ev[0]) e = hipEventRecord(g_fwd_ev[0], s);
  if (e == hipSuccess) e = nc::launch_prologue(pp, bf16, false, s);
  if (e == hipSuccess && g_fwd_ev[1]) e = hipEventRecord(g_fwd_ev[1], s);
  if (e == hipSuccess) {
    nc::FwdParams p{bf16 ? q_raw : q_out, k_out, v, out, lse, B, T, H, Hkv, D, norm_window(window, T), scale,
                    scale * 1.4426950408889634f, nullptr, T, bf16 ? q_out : nullptr, pos_offset, cos_tab, sin_tab,
                    T_rope, eps};
    e = bf16 ? nc::launch_attn_fwd_bf16(p, s) : nc::launch_attn_fwd_f32(p, s);
  }
  if (e == hipSuccess && g_fwd_ev[2]) e = hipEventRecord(g_fwd_ev[2], s);
  return finish(e, s, "nc_attn_fwd_prologue");
}

nc_status nc_profile_fwd_prologue(void* prologue_begin, void* fwd_begin, void* end) {
  const int set = (prologue_begin != nullptr) + (fwd_begin != nullptr) + (end != nullptr);
  if (set != 0 && set != 3) return fail(NC_ERR_INVALID_ARG, "the three events must all be set or all be NULL");
  g_fwd_ev[0] = (hipEvent_t)prologue_begin;
  g_fwd_ev[1] = (hipEvent_t)fwd_begin;
  g_fwd_ev[2] = (hipEvent_t)end;
  g_msg[0] = 0;
  return NC_OK;
}

nc_status nc_measure_shader_clock(unsigned long long* out, int milliseconds, nc_stream stream) {
  NC_TRY(check_ptr(out, "out"));
  if (milliseconds < 1 || milliseconds > 10000)
    return fail(NC_ERR_INVALID_ARG, "milliseconds=%d outside 1..10000", milliseconds);
  NC_TRY(check_device(nullptr));
  hipStream_t s = (hipStream_t)stream;
  return finish(nc::launch_shader_clock(out, 100000ull * (unsigned long long)milliseconds, s), s,
                "nc_measure_shader_clock");
}

nc_status nc_qk_prologue_fwd(nc_dtype dt, int B, int T, int H, int Hkv, int D, const void* q, const void* k,
                             const int32_t* pos_offset, const float* cos_tab, const float* sin_tab, int T_rope,
                             float eps, void* q_out, void* k_out, nc_stream stream) {
  NC_TRY(prologue_common(dt, B, T, H, Hkv, D, q, k, pos_offset, cos_tab, sin_tab, T_rope, eps));
  NC_TRY(check_ptr(q_out, "q_out"));
  NC_TRY(check_ptr(k_out, "k_out"));
  NC_TRY(check_device(nullptr));
  nc::PrologueParams p{q, k, pos_offset, cos_tab, sin_tab, nullptr, nullptr, q_out, k_out, B, T, H, Hkv, D, T_rope, eps};
  hipStream_t s = (hipStream_t)stream;
  return finish(nc::launch_prologue(p, dt == NC_BF16, false, s), s, "nc_qk_prologue_fwd");
}

nc_status nc_qk_prologue_bwd(nc_dtype dt, int B, int T, int H, int Hkv, int D, const void* q, const void* k,
                             const int32_t* pos_offset, const float* cos_tab, const float* sin_tab, int T_rope,
                             float eps, const void* dq_out, const void* dk_out, void* dq, void* dk,
                             nc_stream stream) {
  NC_TRY(prologue_common(dt, B, T, H, Hkv, D, q, k, pos_offset, cos_tab, sin_tab, T_rope, eps));
  NC_TRY(check_ptr(dq_out, "dq_out"));
  NC_TRY(check_ptr(dk_out, "dk_out"));
  NC_TRY(check_ptr(dq, "dq"));
  NC_TRY(check_ptr(dk, "dk"));
  NC_TRY(check_device(nullptr));
  nc::PrologueParams p{q, k, pos_offset, cos_tab, sin_tab, dq_out, dk_out, dq, dk, B, T, H, Hkv, D, T_rope, eps};
  hipStream_t s = (hipStream_t)stream;
  return finish(nc::launch_prologue(p, dt == NC_BF16, true, s), s, "nc_qk_prologue_bwd");
}

}  // extern "C"
