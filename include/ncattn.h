/*
 * libncattn — nanochat's attention hot path for AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every tensor argument is a plain device pointer to memory the caller
 * owns (any HIP device allocation on the current device); sizes are plain
 * ints. The library allocates no device memory, keeps no per-call state and
 * never synchronises: every entry point validates its arguments on the host,
 * enqueues its kernels on the caller's stream and returns. Results are
 * available once the stream has reached that point.
 *
 * Layouts (row-major, innermost dimension last, fully contiguous):
 *   q, out, dq, dout      [B, T, H,   D]
 *   k, v, dk, dv          [B, T, Hkv, D]
 *   lse, delta            [B, H, T]  float32, natural log
 *   decode q, out         [B, H, D];  decode lse [B, H] float32
 *   decode caches         [B, T_max, Hkv, D]  (one layer's slab of a
 *                          (n_layers, B, T_max, Hkv, D) cache)
 * Element type of q/k/v/out/gradients/caches is given by nc_dtype; lse,
 * RoPE tables and workspaces are float32.
 *
 * Grouped-query attention: query head h reads key/value head h / (H / Hkv)
 * ("nanochat Admin & Developer Guide", section 3: n_kv_head <= n_head;
 * section 6: GQA through KV heads repeated in place).
 *
 * Window: key j is visible to query i iff i - window < j <= i, i.e. window
 * counts the keys a query sees including itself; window <= 0 or
 * window >= T means full causal attention (section 3, "Sliding-window
 * attention": per-layer windows handed to the kernel as (left, right)
 * tuples; a (left, 0) tuple is window = left + 1).
 *
 * Errors: validation happens before any HIP call and before any output is
 * touched; on an error nothing is launched and the outputs keep their
 * contents. nc_last_error_message() gives a per-thread description of the
 * last error. Requirements checked: non-null pointers, sizes >= 1,
 * H % Hkv == 0, D in {32, 64, 128}, a known dtype, 16-byte aligned tensor
 * pointers, element counts below 2^31, sufficient workspace, and a gfx950
 * current device (NC_ERR_DEVICE otherwise). Grid limits (NC_ERR_UNSUPPORTED):
 * the float32 attention path takes B, H <= 65535; decode takes B <= 65535
 * and at most 65535 cache chunks (T_max <= 65535 * chunk, the chunk being
 * 64 positions at D = 128 for groups of 1 or 2 heads). A launch failure reported by the
 * runtime gives NC_ERR_LAUNCH; outputs are then undefined. Outputs must not
 * alias inputs. All entry points are thread-safe and reentrant.
 */
#ifndef NCATTN_H
#define NCATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NCATTN_ABI_VERSION 1

typedef enum {
  NC_OK = 0,
  NC_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad window/scale */
  NC_ERR_UNSUPPORTED = 2, /* valid but not built: head dim, dtype, size limit */
  NC_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required */
  NC_ERR_DEVICE = 4,      /* no device, or the current device is not gfx950 */
  NC_ERR_LAUNCH = 5       /* the runtime reported an error after a launch */
} nc_status;

typedef enum { NC_F32 = 0, NC_BF16 = 1 } nc_dtype;

/* A hipStream_t (NULL = the default stream); kept opaque so that callers do
 * not need HIP headers. */
typedef void* nc_stream;

int nc_abi_version(void);
const char* nc_status_string(nc_status s);
/* Description of the last error on the calling thread ("" if none). */
const char* nc_last_error_message(void);

/*
 * Attention forward.
 * Computes, per (b, h) with g = h / (H / Hkv) and s_ij = scale * <q_i, k_j>:
 *   lse_i = ln sum_{j visible} exp(s_ij),  out_i = sum_{j visible} exp(s_ij - lse_i) v_j.
 * Defined by "nanochat Admin & Developer Guide", section 3 (causal GQA with
 * per-layer sliding windows) and section 6 (the FA3 / SDPA attention call).
 * bf16: inputs bf16, products on bf16 matrix cores with float32 accumulation,
 * softmax statistics in float32, probabilities rounded to bf16 before the
 * P.V product, out rounded to nearest even. f32: float32 throughout.
 *   q [B,T,H,D], k/v [B,T,Hkv,D] (dtype dt)  -> out [B,T,H,D] (dt), lse [B,H,T] (f32)
 * scale must be finite and > 0.
 */
nc_status nc_attn_fwd(nc_dtype dt, int B, int T, int H, int Hkv, int D,
                      const void* q, const void* k, const void* v,
                      int window, float scale,
                      void* out, float* lse, nc_stream stream);

/*
 * Attention forward of fp8 operands ("nanochat Admin & Developer Guide",
 * section 5 "Precision: Explicit dtype & FP8": forward operands in float8
 * e4m3 with tensorwise scaling; section 6: the attention kernel accepts fp8
 * as well as bf16). q, k, v are float8 e4m3 codes in the OCP "fn" encoding
 * (1 byte per element, no infinities), each tensor with one descale: the
 * operands are q = value(q8) * q_descale, likewise k, v. Computes the
 * forward of nc_attn_fwd on those values:
 *   q8 [B,T,H,D], k8/v8 [B,T,Hkv,D] (bytes) -> out [B,T,H,D] bf16, lse [B,H,T] f32
 * Products on the 32x32x64 fp8 matrix cores with float32 accumulation,
 * softmax statistics in float32; the probabilities are rounded to e4m3
 * (round to nearest even) before the P.V product. D in {64, 128}
 * (NC_ERR_UNSUPPORTED otherwise); scale and the descales must be finite and
 * > 0, NC_ERR_INVALID_ARG otherwise. Pointers 16-byte aligned.
 */
nc_status nc_attn_fwd_fp8(int B, int T, int H, int Hkv, int D, const void* q8, const void* k8,
                          const void* v8, float q_descale, float k_descale, float v_descale,
                          int window, float scale, void* out, float* lse, nc_stream stream);

/*
 * A chunk of Tq queries per row against a KV cache: the SDPA fallback's
 * chunked-inference case ("nanochat Admin & Developer Guide", section 6: the
 * queries are fewer than the keys and the visible keys are a shifted causal,
 * optionally windowed, band; section 7 "KV cache": per-row int32
 * cache_seqlens). Row b holds n = cache_seqlens[b] tokens before the chunk;
 * the chunk's keys and values must already be in cache slots n .. n + Tq - 1
 * (nc_kv_cache_append). Chunk query t sits at position p = n + t and sees
 * slots j with p - window < j <= p (window <= 0: all j <= p):
 *   lse[b,h,t] = ln sum_j exp(s_tj),  out[b,t,h] = sum_j exp(s_tj - lse) v_j,
 *   s_tj = scale * <q[b,t,h], k_cache[b,j,g]>.
 * Same kernels and numerics as nc_attn_fwd (which is this call with n = 0,
 * Tq = T_max = T). cache_seqlens is a DEVICE int32 array [B]; a row with
 * n < 0 or n + Tq > T_max gets NaN out and lse. Keys are read in tiles of 64
 * positions and masked, so slots 0 .. n + Tq - 1 must hold finite values
 * (as they do once earlier steps have filled them); later slots are not read.
 *   q [B,Tq,H,D] (after the prologue, e.g. nc_qk_prologue_fwd with
 *   pos_offset = cache_seqlens), k_cache/v_cache [B,T_max,Hkv,D]
 *   -> out [B,Tq,H,D], lse [B,H,Tq]
 */
nc_status nc_attn_fwd_cache(nc_dtype dt, int B, int Tq, int H, int Hkv, int D, int T_max,
                            const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* cache_seqlens, int window, float scale,
                            void* out, float* lse, nc_stream stream);

/*
 * Writes a chunk's keys and values into the cache in place (section 7 "KV
 * cache"): k_cache[b, n + t] <- k_new[b, t], v_cache[b, n + t] <- v_new[b, t]
 * for t < Tq, n = cache_seqlens[b] (DEVICE int32 [B], not modified). A row
 * with n < 0 or n + Tq > T_max is left untouched. Nothing else is written.
 *   k_new/v_new [B,Tq,Hkv,D] -> k_cache/v_cache [B,T_max,Hkv,D]
 */
nc_status nc_kv_cache_append(nc_dtype dt, int B, int Tq, int Hkv, int D, int T_max,
                             const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* cache_seqlens, nc_stream stream);

/*
 * Attention backward: gradients of L = sum(out * dout) w.r.t. q, k, v, with
 * P recomputed from the saved lse. Per (b, h):
 *   dP_ij = <dout_i, v_j>, delta_i = <dout_i, out_i>,
 *   dS_ij = P_ij (dP_ij - delta_i),
 *   dq_i = scale sum_j dS_ij k_j,
 *   dk_j = scale sum_{h in group} sum_i dS_ij q_i,
 *   dv_j = sum_{h in group} sum_i P_ij dout_i.
 * dk/dv are summed over the query heads of each group. dq/dk/dv are fully
 * overwritten. q, k, v, out, lse must be those of nc_attn_fwd with the same
 * window and scale.
 * Defined by the attention call it differentiates ("nanochat Admin &
 * Developer Guide", section 6 "Attention: FA3 with SDPA Fallback": causal
 * GQA with the layer's window; section 3: the sliding-window schedule) and
 * by the pages' statement that upstream takes this gradient with autograd
 * ("nanochat (Python)" catalog, "Model & kernels"): the formulas above are
 * the chain rule through the softmax, loss convention L = sum(out * dout).
 * bf16: products on bf16 matrix cores with float32 accumulation, P and dS
 * rounded to bf16 before the products that consume them, gradients rounded
 * to nearest even. f32: float32 throughout.
 *   q, out, dout [B,T,H,D], k, v [B,T,Hkv,D] (dt), lse [B,H,T] (f32)
 *   -> dq [B,T,H,D], dk, dv [B,T,Hkv,D] (dt)
 * workspace: caller-owned DEVICE memory of at least
 * nc_attn_bwd_workspace_bytes() bytes, 16-byte aligned; it holds float32
 * delta [B,H,T] and lse*log2(e) [B,H,T] (each padded to 256 bytes), is
 * fully overwritten, and carries nothing between calls (NC_ERR_WORKSPACE if
 * NULL or smaller). Calls that share a workspace must be ordered on one
 * stream. dq, dk and dv are deterministic (no atomics; dq comes from its own
 * query-stationary pass). Errors as in the header comment.
 */
/* Bytes of workspace nc_attn_bwd and nc_attn_bwd_prologue need for these
 * sizes (section 6's attention call and its backward, as above); a pure
 * function of its arguments, 0 for invalid sizes. */
size_t nc_attn_bwd_workspace_bytes(nc_dtype dt, int B, int T, int H, int Hkv, int D);
nc_status nc_attn_bwd(nc_dtype dt, int B, int T, int H, int Hkv, int D,
                      const void* q, const void* k, const void* v,
                      const void* out, const float* lse, const void* dout,
                      int window, float scale,
                      void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, nc_stream stream);

/*
 * Backward through attention and the QK prologue in one call: the result of
 * nc_attn_bwd followed by nc_qk_prologue_bwd, i.e. dq, dk are gradients
 * w.r.t. the raw q_raw, k_raw ("nanochat Admin & Developer Guide", section 3:
 * q and k are RMS-normalised and rotated before attention; the gradient
 * passes back through both). q, k are the prologue outputs given to
 * nc_attn_fwd; v, out, lse, dout, window, scale, workspace as for
 * nc_attn_bwd; q_raw, k_raw, pos_offset, cos_tab, sin_tab, T_rope, eps as
 * for nc_qk_prologue_bwd. For bf16 the prologue backward is applied by the
 * backward kernels as they store dq and dk (the gradients w.r.t. q, k never
 * reach memory). Outputs must not alias inputs. Validation and errors as for
 * both calls it combines.
 */
nc_status nc_attn_bwd_prologue(nc_dtype dt, int B, int T, int H, int Hkv, int D,
                               const void* q, const void* k, const void* v,
                               const void* out, const float* lse, const void* dout,
                               int window, float scale,
                               const void* q_raw, const void* k_raw, const int32_t* pos_offset,
                               const float* cos_tab, const float* sin_tab, int T_rope, float eps,
                               void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, nc_stream stream);

/*
 * Measurement aid. While set on the calling thread, every nc_attn_bwd call
 * records, on its stream, dq_begin just before the kernel that forms dQ
 * (for bf16 it also forms the row statistics), dkdv_begin between it and
 * the kernel that forms dK and dV, and end just after that one, so a caller
 * can time each kernel alone with hipEventElapsedTime. All are hipEvent_t
 * created by the caller; passing NULL for all three clears the setting.
 * Returns NC_ERR_INVALID_ARG unless all three or none are NULL.
 */
nc_status nc_profile_bwd_main(void* dq_begin, void* dkdv_begin, void* end);
/* (nc_attn_bwd_prologue records the same events.) */

/*
 * Single-token decode against one layer's KV cache ("nanochat Admin &
 * Developer Guide", section 7 "KV cache": per-layer (B, T, H, D) cache with
 * int32 per-row lengths; section 6: single-token decode slices the key
 * window). Row b holds seqlens[b] cached keys including the current token,
 * whose query sits at position seqlens[b] - 1; it sees cache positions
 * max(0, seqlens[b] - window) .. seqlens[b] - 1 (all of them when
 * window <= 0 or window >= seqlens[b]). Positions outside that range are never
 * read. seqlens is a DEVICE int32 array [B]; values outside 1..T_max cannot
 * be checked without a sync, so such a row's out and lse are written as NaN.
 *   q [B,H,D], k_cache/v_cache [B,T_max,Hkv,D], seqlens [B]
 *   -> out [B,H,D], lse [B,H]
 * The float32 workspace holds split-K partials; size from
 * nc_attn_decode_workspace_bytes().
 */
size_t nc_attn_decode_workspace_bytes(nc_dtype dt, int B, int H, int Hkv, int D, int T_max);
nc_status nc_attn_decode(nc_dtype dt, int B, int H, int Hkv, int D, int T_max,
                         const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seqlens, int window, float scale,
                         void* out, float* lse,
                         void* workspace, size_t workspace_bytes, nc_stream stream);

/*
 * One decode step of one layer with the cache updated in place, the way the
 * pages describe the engine's use of FA3's kvcache call ("nanochat Admin &
 * Developer Guide", section 7 "KV cache": the position of each row is its
 * int32 cache_seqlens entry and the cache is written in place; section 3:
 * the QK prologue, RMSNorm without weights then half-split RoPE).
 * Row b holds n = cache_seqlens[b] cached tokens; the new token sits at
 * position n:
 *   q' = RoPE(RMSNorm(q[b]), n),  k' = RoPE(RMSNorm(k_new[b]), n)
 *   k_cache[b, n] <- k',  v_cache[b, n] <- v_new[b]      (every kv head)
 *   out[b], lse[b] = attention of q' over cache positions
 *                    max(0, n + 1 - window) .. n        (window <= 0: all)
 * exactly as nc_attn_decode with seqlens[b] = n + 1. cache_seqlens is a
 * DEVICE int32 array [B] and is not modified (the caller advances it).
 * A row with n outside 0..min(T_max, T_rope) - 1 leaves the cache untouched
 * and gets NaN out and lse. Nothing else in the cache is written.
 *   q [B,H,D], k_new/v_new [B,Hkv,D] (raw, before the prologue),
 *   k_cache/v_cache [B,T_max,Hkv,D] (read and written), cos/sin [T_rope,D/2]
 *   -> out [B,H,D], lse [B,H]
 * k' is stored in the cache's dtype and the attention reads that stored
 * value; q' is rounded to that dtype too, as the prologue's output is in the
 * forward (nc_attn_fwd_prologue), so the step attends like the last row of a
 * prefill of the same tokens. The inputs must not overlap the caches. The
 * workspace (size from nc_attn_decode_step_workspace_bytes, the same as
 * nc_attn_decode's) holds the split-K partials.
 */
size_t nc_attn_decode_step_workspace_bytes(nc_dtype dt, int B, int H, int Hkv, int D, int T_max);
nc_status nc_attn_decode_step(nc_dtype dt, int B, int H, int Hkv, int D, int T_max,
                              const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const int32_t* cache_seqlens,
                              const float* cos_tab, const float* sin_tab, int T_rope, float eps,
                              int window, float scale, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, nc_stream stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the step
 * of nc_attn_decode_step, same arguments, results and errors, without the
 * workspace. Its split-K partials go to a scratch array that the library
 * holds on each GPU it runs on (NC_NOALLOC_SCRATCH_BYTES, placed when the
 * library's code is loaded on that GPU and kept until the process ends);
 * this call allocates nothing. Sizes whose partials
 * (nc_attn_decode_step_workspace_bytes) exceed that array give
 * NC_ERR_UNSUPPORTED with nothing launched. Every call on a GPU shares that
 * GPU's array and leaves its partials there: calls that may overlap on one
 * GPU (e.g. on two streams without ordering between them) race and must not
 * be issued; calls ordered on one stream are safe. Nothing in the array
 * needs to start at zero (each call writes every partial it reads).
 */
#define NC_NOALLOC_SCRATCH_BYTES (32u << 20)
nc_status nc_attn_decode_step_noalloc(nc_dtype dt, int B, int H, int Hkv, int D, int T_max,
                                      const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int32_t* cache_seqlens,
                                      const float* cos_tab, const float* sin_tab, int T_rope, float eps,
                                      int window, float scale, void* out, float* lse, nc_stream stream);

/*
 * Expands a batch-1 prefill cache into a decode cache of n_rows rows, so the
 * prompt is processed once ("nanochat Admin & Developer Guide", section 7
 * "KV cache" and "Generation flow": prefill once, then replicate the cache
 * across the samples). Copies positions 0..n_tokens-1 of src (one row,
 * position-major [>= n_tokens, Hkv, D]) into rows 0..n_rows-1 of
 * dst [n_rows, T_max, Hkv, D]; later positions of dst are not written.
 * Call once for k and once for v of each layer; src and dst must not overlap.
 */
nc_status nc_kv_cache_replicate(nc_dtype dt, int n_rows, int T_max, int Hkv, int D, int n_tokens,
                                const void* src, void* dst, nc_stream stream);

/*
 * RoPE table: cos_out[p, d] = cos(p * base^(-2d/D)), sin_out likewise, for
 * p in 0..T_rope-1 and d in 0..D/2-1, float32 [T_rope, D/2]. Angles and the
 * trigonometry are evaluated in float64 on the device, then rounded to
 * float32. ("nanochat Admin & Developer Guide", section 3: rotary
 * embeddings with base 100000, table over-computed past the sequence
 * length; "nanochat (Fucina port)", "Architecture": table built from the
 * inverse frequencies.) base must be > 1; D even, 2..256.
 */
nc_status nc_rope_table(int T_rope, int D, double base,
                        float* cos_out, float* sin_out, nc_stream stream);

/*
 * QK prologue forward: for every head vector x (of q and of k) at position
 * p = (pos_offset ? pos_offset[b] : 0) + t:
 *   y = x / sqrt(mean_d x_d^2 + eps)                (RMSNorm, no weight)
 *   (y_d, y_{d+D/2}) <- (y_d c - y_{d+D/2} s, y_d s + y_{d+D/2} c),  d < D/2,
 *   c = cos[p, d], s = sin[p, d]                    (half-split RoPE)
 * ("nanochat Admin & Developer Guide", section 3: QK-norm without learnable
 * parameters, RoPE; "nanochat (Fucina port)", "Architecture"). Statistics in
 * float32. pos_offset is a DEVICE int32 array [B] or NULL; a position
 * outside 0..T_rope-1 writes NaN for that vector.
 *   q [B,T,H,D], k [B,T,Hkv,D] -> q_out, k_out (same shape and dtype)
 */
nc_status nc_qk_prologue_fwd(nc_dtype dt, int B, int T, int H, int Hkv, int D,
                             const void* q, const void* k, const int32_t* pos_offset,
                             const float* cos_tab, const float* sin_tab, int T_rope,
                             float eps, void* q_out, void* k_out, nc_stream stream);

/*
 * QK prologue and attention forward in one call: the result of
 * nc_qk_prologue_fwd (q_out = q', k_out = k') followed by nc_attn_fwd on q',
 * k', v ("nanochat Admin & Developer Guide", section 3: q and k are
 * RMS-normalised and rotated right before attention). For bf16 the keys go
 * through the prologue kernel alone and the forward kernel applies the
 * prologue to each query row as it loads it, storing q' (the backward needs
 * q' and k'); q' and k' are the bf16 values the attention uses. The row sums
 * of squares are added in a different order than the prologue kernel's, so
 * q_out may differ from nc_qk_prologue_fwd's by one bf16 rounding in rare
 * elements. Arguments as for nc_qk_prologue_fwd and nc_attn_fwd; outputs
 * must not alias inputs.
 */
nc_status nc_attn_fwd_prologue(nc_dtype dt, int B, int T, int H, int Hkv, int D,
                               const void* q_raw, const void* k_raw, const void* v,
                               const int32_t* pos_offset, const float* cos_tab,
                               const float* sin_tab, int T_rope, float eps,
                               int window, float scale, void* q_out, void* k_out,
                               void* out, float* lse, nc_stream stream);

/*
 * Measurement aid, like nc_profile_bwd_main: while set on the calling thread,
 * every nc_attn_fwd_prologue call records prologue_begin before its prologue
 * kernel, fwd_begin between it and the forward kernel, and end after that.
 * All three hipEvent_t or none (NULL clears); NC_ERR_INVALID_ARG otherwise.
 */
nc_status nc_profile_fwd_prologue(void* prologue_begin, void* fwd_begin, void* end);

/*
 * Measurement aid: launches one wave on `stream` that runs for `milliseconds`
 * of wall time (by the GPU's constant 100 MHz counter) and then writes
 * out[0] = shader-clock cycles and out[1] = 100 MHz ticks that passed, as
 * uint64 to DEVICE memory `out` (2 values, caller-owned). Enqueued on a
 * second stream while other kernels run, out[0] / out[1] * 100 MHz is the
 * average shader clock they ran at; the wave sleeps between counter reads.
 * NC_ERR_INVALID_ARG for a NULL out or milliseconds outside 1..10000.
 */
nc_status nc_measure_shader_clock(unsigned long long* out, int milliseconds, nc_stream stream);

/*
 * QK prologue backward: given dq_out, dk_out (gradients w.r.t. the prologue
 * outputs) and the raw q, k, writes dq, dk w.r.t. the raw inputs:
 *   u = R(-theta) dy,  r = sqrt(mean x^2 + eps),  dx = u / r - x <x, u> / (D r^3).
 * It differentiates nc_qk_prologue_fwd ("nanochat Admin & Developer Guide",
 * section 3: weightless QK RMSNorm then half-split RoPE with base 100000,
 * applied to q and k right before attention; the pages take this gradient
 * with autograd, "nanochat (Python)" catalog, "Model & kernels"): the
 * transpose of the rotation by theta = p * base^(-2d/D), then the
 * transposed Jacobian of the norm, d(x_i/r)/dx_k = delta_ik/r - x_i x_k/(D r^3).
 * Positions p = (pos_offset ? pos_offset[b] : 0) + t as in the forward
 * (pos_offset a DEVICE int32 array [B] or NULL); a position outside
 * 0..T_rope-1 writes NaN for that vector. Statistics in float32, results
 * rounded to the dtype.
 *   q, dq_out [B,T,H,D], k, dk_out [B,T,Hkv,D] (raw inputs and incoming
 *   gradients, dtype dt), cos/sin [T_rope,D/2] f32
 *   -> dq [B,T,H,D], dk [B,T,Hkv,D] (dt)
 * Outputs must not alias inputs. Errors as in the header comment.
 */
nc_status nc_qk_prologue_bwd(nc_dtype dt, int B, int T, int H, int Hkv, int D,
                             const void* q, const void* k, const int32_t* pos_offset,
                             const float* cos_tab, const float* sin_tab, int T_rope,
                             float eps, const void* dq_out, const void* dk_out,
                             void* dq, void* dk, nc_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* NCATTN_H */
