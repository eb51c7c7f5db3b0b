// Kernel parameter blocks and launchers (internal to libncattn).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nc {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  int B, T, H, Hkv, D;
  int window;        // 0 = full causal, otherwise 1 <= window < T
  float scale;       // logit scale
  float scale_log2;  // scale * log2(e)
  // Chunk against a cache (q_off != nullptr): q/out hold T chunk rows per
  // batch row, k/v are caches of T_kv positions per batch row, and chunk row
  // t of batch row b sits at position q_off[b] + t, seeing cache positions
  // up to that one. Without it T_kv == T and positions are the rows.
  const int32_t* q_off;
  int T_kv;
  // Query prologue in the forward (q_out != nullptr, bf16, no cache): q holds
  // the raw queries; each row gets RMSNorm + RoPE at position
  // (pos_offset ? pos_offset[b] : 0) + t as it is loaded, and q' goes to q_out.
  void* q_out;
  const int32_t* pos_offset;
  const float* cos_tab;  // [T_rope, D/2]
  const float* sin_tab;
  int T_rope;
  float eps;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* delta;   // [B, H, T] workspace
  float* lse2;    // [B, H, T] workspace: lse * log2(e)
  int B, T, H, Hkv, D;
  int window;
  float scale;
  float scale_log2;
  // Optional QK prologue backward applied to dq and dk before they are
  // stored (q_raw == nullptr: dq, dk are the gradients w.r.t. q, k).
  const void* q_raw;
  const void* k_raw;
  const int32_t* pos_offset;  // device [B] or nullptr
  const float* cos_tab;       // [T_rope, D/2]
  const float* sin_tab;
  int T_rope;
  float eps;
};

struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* seqlens;
  void* out;
  float* lse;
  float* part;  // [B, H, n_split, D + 2] workspace (acc[D], m, l)
  int B, H, Hkv, D, T_max;
  int window;  // <= 0 full
  int n_split;
  float scale;
  float scale_log2;
  // Decode step (step != 0): q [B,H,D], k_new, v_new [B,Hkv,D] are raw, in
  // the cache dtype; seqlens[b] counts the tokens already cached (the new
  // one goes to slot n = seqlens[b] and the row attends to n + 1 keys). The
  // kernels apply the prologue at position n and write k', v into the slot.
  int step;
  const void* k_new;
  const void* v_new;
  const float* cos_tab;  // [T_rope, D/2]
  const float* sin_tab;
  int T_rope;
  float eps;
};

struct PrologueParams {
  const void* q;
  const void* k;
  const int32_t* pos_offset;
  const float* cos_tab;
  const float* sin_tab;
  const void* dq_out;  // backward only
  const void* dk_out;  // backward only
  void* q_out;         // forward: q'; backward: dq
  void* k_out;         // forward: k'; backward: dk
  int B, T, H, Hkv, D, T_rope;
  float eps;
};

// Decode: cache positions per group of D/8 lanes for a query group of G heads
// (fewer when several heads share the scores' registers), and positions per
// wave (one wave per (row, kv head, chunk)).
constexpr int decode_keys_per_group(int G) { return G <= 2 ? 16 : (G <= 4 ? 8 : 4); }
constexpr int decode_chunk(int D, int G) { return (64 / (D / 8)) * decode_keys_per_group(G); }

// Forward of float8 e4m3 operands (one descale per tensor), bf16 out.
struct Fp8FwdParams {
  const void* q;  // e4m3 codes [B, T, H, D]
  const void* k;  // [B, T, Hkv, D]
  const void* v;
  void* out;      // bf16 [B, T, H, D]
  float* lse;     // [B, H, T], natural log of the scaled scores
  int B, T, H, Hkv, D;
  int window;        // 0 = full causal, otherwise 1 <= window < T
  float scale_log2;  // scale * q_descale * k_descale * log2(e)
  float v_descale;
};
hipError_t launch_attn_fwd_fp8(const Fp8FwdParams& p, hipStream_t s);

// Average shader clock: out[0] shader cycles and out[1] 100 MHz ticks over
// `ticks` ticks of wall time (device memory, 2 values).
hipError_t launch_shader_clock(unsigned long long* out, unsigned long long ticks, hipStream_t s);

hipError_t launch_attn_fwd_bf16(const FwdParams& p, hipStream_t s);
hipError_t launch_attn_fwd_f32(const FwdParams& p, hipStream_t s);
// Optional events (null = not recorded): before the dQ kernel, between it
// and the dK/dV kernel, and after the dK/dV kernel.
struct BwdEvents {
  hipEvent_t dq_begin, dkdv_begin, end;
};
hipError_t launch_attn_bwd_bf16(const BwdParams& p, hipStream_t s, const BwdEvents& ev);
hipError_t launch_attn_bwd_f32(const BwdParams& p, hipStream_t s, const BwdEvents& ev);
hipError_t launch_decode(const DecodeParams& p, bool bf16, hipStream_t s);
// Chunk k/v [B, Tq, Hkv, D] into cache slots cache_seqlens[b] .. + Tq - 1 (rows
// whose slots do not fit are left alone).
hipError_t launch_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const int32_t* cache_seqlens, int B, int Tq, int Hkv, int D, int T_max,
                               size_t elem_bytes, hipStream_t s);
// Copies the first n_bytes of src into n_rows rows of dst spaced row_stride bytes apart.
hipError_t launch_replicate(const void* src, void* dst, size_t n_bytes, int n_rows, size_t row_stride, hipStream_t s);
hipError_t launch_rope_table(int T_rope, int D, double base, float* c, float* sn, hipStream_t s);
hipError_t launch_prologue(const PrologueParams& p, bool bf16, bool backward, hipStream_t s);

}  // namespace nc
