// Single-token KV-cache decode for gfx950 (split-K over ragged lengths).
//
// Row b holds L_b = seqlens[b] cached keys including the current token; its
// query sits at position L_b - 1 and attends to cache positions
// max(0, L_b - w) .. L_b - 1 (all of them for a full-context layer).
// ("nanochat Admin & Developer Guide", section 7 "KV cache": per-layer
// (B, T, H, D) cache, per-row int32 lengths; section 6: single-token decode
// slices the key window.)
//
// decode_split: one wave per (kv head, chunk of cache positions, row), kv
//   heads fastest in the grid so that the waves dispatched together read the
//   whole of each cache position (its Hkv head rows are contiguous). The
//   wave's groups of D/8 lanes each take every NGR-th position of the chunk,
//   so one load instruction reads NGR whole head vectors (256 bytes each at
//   D = 128). All of a group's K and V rows are requested before any is used
//   (one memory round trip per wave), the dot products are finished with DPP
//   exchanges inside the group, the softmax is taken in one pass over the
//   known scores, and the groups are merged with DPP row rotations and
//   permlane swaps (no LDS traffic). One partial (acc[D], m, l) per
//   (row, query head, chunk) goes to the workspace.
//   Chunks outside a row's key range exit without reading anything.
// decode_combine: merges a row's partials into out and lse. A length outside
//   1..T_max yields NaN out and lse for that row.
// Decode step (the in-place cache update of FA3's kvcache call that the
//   pages describe: section 7, per-row int32 cache_seqlens): row b holds
//   n = cache_seqlens[b] cached tokens and the new token sits at position n.
//   The split kernel applies the forward prologue at position n to the raw
//   q and to the raw new key, both rounded to the cache dtype as the
//   prologue's outputs are in the forward; the wave whose chunk holds
//   position n uses the new k' (rounded to the cache dtype) and v for that
//   position and writes both into cache slot n. A row whose n is outside
//   0 .. min(T_max, T_rope) - 1 writes nothing and gets NaN out and lse.
// replicate: copies a batch-1 prompt cache row into every decode row (section
//   7: the prompt is prefilled once and its cache copied to the samples).
// cache_append: writes a chunk's k and v into the cache slots that follow
//   each row's cached tokens (the in-place update of section 7, for a chunk).

#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "rope.hpp"

namespace nc {
namespace {

// 8 elements of a cache row as loaded (bf16: 16 bytes, float32: 32 bytes)
template <bool BF16>
struct Raw8 {
  u32x4 w[BF16 ? 1 : 2];
};
template <bool BF16>
__device__ __forceinline__ Raw8<BF16> load_raw8(const void* base, size_t elem_off) {
  Raw8<BF16> r;
  if (BF16) {
    r.w[0] = __builtin_nontemporal_load((const u32x4*)((const unsigned short*)base + elem_off));
  } else {
    const u32x4* p = (const u32x4*)((const float*)base + elem_off);
    r.w[0] = __builtin_nontemporal_load(p);
    r.w[BF16 ? 0 : 1] = __builtin_nontemporal_load(p + 1);
  }
  return r;
}
template <bool BF16>
__device__ __forceinline__ void unpack_raw8(const Raw8<BF16>& r, float* f) {
  if (BF16) {
    unpack8_bf16(r.w[0], f);
  } else {
    const f32x4 a = __builtin_bit_cast(f32x4, r.w[0]), b = __builtin_bit_cast(f32x4, r.w[BF16 ? 0 : 1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  }
}

// Keys row b attends to (its query sits at position keys - 1); a value
// outside 1..T_max marks the row invalid.
__device__ __forceinline__ int row_keys(const DecodeParams& p, int b) {
  const int n = p.seqlens[b];
  if (!p.step) return n;
  return (n >= 0 && n < p.T_max && n < p.T_rope) ? n + 1 : 0;
}

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> to_raw8(const float* f) {
  Raw8<BF16> r;
  if (BF16) {
    r.w[0] = pack8_bf16(f);
  } else {
    r.w[0] = __builtin_bit_cast(u32x4, (f32x4){f[0], f[1], f[2], f[3]});
    r.w[BF16 ? 0 : 1] = __builtin_bit_cast(u32x4, (f32x4){f[4], f[5], f[6], f[7]});
  }
  return r;
}
template <bool BF16>
__device__ __forceinline__ void store_raw8(const void* base, size_t elem_off, const Raw8<BF16>& r) {
  if (BF16) {
    *(u32x4*)((unsigned short*)const_cast<void*>(base) + elem_off) = r.w[0];
  } else {
    u32x4* d = (u32x4*)((float*)const_cast<void*>(base) + elem_off);
    d[0] = r.w[0];
    d[1] = r.w[BF16 ? 0 : 1];
  }
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeParams p) {
  constexpr int LPR = D / 8;              // lanes per cache row (divides 16)
  constexpr int NGR = 64 / LPR;           // row groups per wave
  constexpr int KPG = decode_keys_per_group(G);
  constexpr int CHUNK = NGR * KPG;        // positions per wave
  static_assert(CHUNK == decode_chunk(D, G), "chunk size mismatch");

  const int g = blockIdx.x, sp = blockIdx.y, b = blockIdx.z;
  const int L = row_keys(p, b);
  if (L < 1 || L > p.T_max) return;
  const bool full = p.window <= 0 || p.window >= L;
  const int lo = full ? 0 : L - p.window;
  const int k_begin = max(lo, sp * CHUNK);
  const int k_end = min(L, (sp + 1) * CHUNK);  // exclusive
  if (k_begin >= k_end) return;

  const int lane = threadIdx.x;
  const int grp = lane / LPR, c = lane - (lane / LPR) * LPR;
  const int H = p.H;
  const size_t rs = (size_t)p.Hkv * D;  // elements per cache position
  const size_t cache_base = (size_t)b * p.T_max * rs + (size_t)g * D + c * 8;

  // positions sp*CHUNK + grp + NGR*u, u = 0 .. KPG-1 (only those in [k_begin, k_end))
  const int j0 = sp * CHUNK + grp;
  Raw8<BF16> kr[KPG], vr[KPG];
#pragma unroll
  for (int u = 0; u < KPG; ++u) {
    const int j = j0 + NGR * u;
    if (j >= k_begin && j < k_end) {
      kr[u] = load_raw8<BF16>(p.k_cache, cache_base + (size_t)j * rs);
      vr[u] = load_raw8<BF16>(p.v_cache, cache_base + (size_t)j * rs);
    } else {
#pragma unroll
      for (int i = 0; i < (BF16 ? 1 : 2); ++i) {
        kr[u].w[i] = (u32x4){0u, 0u, 0u, 0u};
        vr[u].w[i] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  }

  // decode step: in the wave whose chunk holds position n, the new token's
  // k' and v (every group computes the same vector, all lanes active for the
  // group exchanges) replace what the cache slot held and are written there
  float cs[8], sn[8];
  if (p.step) load_angles8<D>(p.cos_tab, p.sin_tab, L - 1, c, cs, sn);
  if (p.step && sp == (L - 1) / CHUNK) {
    const int n = L - 1;
    float x[8], kp[8];
    ld8<BF16>(p.k_new, ((size_t)b * p.Hkv + g) * D + c * 8, x);
    prologue8<D>(x, cs, sn, c, p.eps, kp);
    const Raw8<BF16> knew = to_raw8<BF16>(kp);
    const Raw8<BF16> vnew = load_raw8<BF16>(p.v_new, ((size_t)b * p.Hkv + g) * D + c * 8);
#pragma unroll
    for (int u = 0; u < KPG; ++u)
      if (j0 + NGR * u == n) {
        kr[u] = knew;
        vr[u] = vnew;
      }
    if (grp == 0) {
      store_raw8<BF16>(p.k_cache, cache_base + (size_t)n * rs, knew);
      store_raw8<BF16>(p.v_cache, cache_base + (size_t)n * rs, vnew);
    }
  }

#pragma unroll
  for (int hq = 0; hq < G; ++hq) {
    float qf[8];
    {
      float t[8];
      if (p.step) {  // raw q in the cache dtype: the prologue at position n, q' rounded to that dtype
        float x[8];
        ld8<BF16>(p.q, ((size_t)b * H + g * G + hq) * D + c * 8, x);
        prologue8<D>(x, cs, sn, c, p.eps, t);
        if (BF16) unpack8_bf16(pack8_bf16(t), t);
      } else if (BF16)
        unpack8_bf16(*(const u32x4*)((const unsigned short*)p.q + ((size_t)b * H + g * G + hq) * D + c * 8), t);
      else {
        const f32x4* pq = (const f32x4*)((const float*)p.q + ((size_t)b * H + g * G + hq) * D + c * 8);
        const f32x4 a = pq[0], bq = pq[1];
        for (int i = 0; i < 4; ++i) {
          t[i] = a[i];
          t[4 + i] = bq[i];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[e] = t[e] * p.scale_log2;
    }
    // scores of the group's positions (log2 units), -inf where absent
    float s[KPG];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      const int j = j0 + NGR * u;
      float kf[8];
      unpack_raw8<BF16>(kr[u], kf);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qf[e], kf[e], d);
      d = group_sum<LPR>(d);
      s[u] = (j >= k_begin && j < k_end) ? d : -INFINITY;
      m = fmaxf(m, s[u]);
    }
    // the wave's maximum (at least one position is present), then one pass
    m = max_mod<LPR>(m);
    float l = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KPG; ++u) {
      const float pe = exp2_fast(s[u] - m);  // 0 for absent positions (their v is 0)
      l += pe;
      float vf[8];
      unpack_raw8<BF16>(vr[u], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(pe, vf[e], acc[e]);
    }
    l = sum_mod<LPR>(l);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = sum_mod<LPR>(acc[e]);
    if (grp == 0) {
      float* dst = p.part + (((size_t)b * H + g * G + hq) * p.n_split + sp) * (D + 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[c * 8 + e] = acc[e];
      if (c == 0) {
        dst[D] = m;
        dst[D + 1] = l;
      }
    }
  }
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeParams p) {
  constexpr int CHUNK = decode_chunk(D, G);
  constexpr int MAXS = 32;  // chunks merged per batch (T_max / CHUNK beyond this loops)
  __shared__ float sm[MAXS], sl[MAXS];
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int L = row_keys(p, b);
  const size_t oi = ((size_t)b * p.H + h) * D + t;
  if (L < 1 || L > p.T_max) {
    if (BF16)
      ((unsigned short*)p.out)[oi] = 0x7fc0;
    else
      ((float*)p.out)[oi] = NAN;
    if (t == 0) p.lse[(size_t)b * p.H + h] = NAN;
    return;
  }
  const bool full = p.window <= 0 || p.window >= L;
  const int lo = full ? 0 : L - p.window;
  const int s0 = lo / CHUNK, s1 = (L - 1) / CHUNK;
  const float* part = p.part + ((size_t)b * p.H + h) * p.n_split * (D + 2);
  // Per batch of up to MAXS chunks, each thread requests its element of
  // every chunk's acc and (threads < nc) one chunk's (m, l) together: one
  // memory round trip; the merge then runs out of registers and LDS.
  float M = -INFINITY, a = 0.f, z = 0.f;
  for (int c0 = s0; c0 <= s1; c0 += MAXS) {
    const int nc = min(MAXS, s1 - c0 + 1);
    float av[MAXS];
#pragma unroll
    for (int i = 0; i < MAXS; ++i) av[i] = i < nc ? part[(size_t)(c0 + i) * (D + 2) + t] : 0.f;
    __syncthreads();  // the previous batch's (m, l) are no longer read
    if (t < nc) {
      sm[t] = part[(size_t)(c0 + t) * (D + 2) + D];
      sl[t] = part[(size_t)(c0 + t) * (D + 2) + D + 1];
    }
    __syncthreads();
    float Mc = -INFINITY;
    for (int i = 0; i < nc; ++i) Mc = fmaxf(Mc, sm[i]);
    const float Mn = fmaxf(M, Mc);
    const float r = exp2_fast(M - Mn);  // 0 on the first batch
    a *= r;
    z *= r;
    M = Mn;
#pragma unroll
    for (int i = 0; i < MAXS; ++i)
      if (i < nc) {
        const float f = exp2_fast(sm[i] - M);
        a = fmaf(f, av[i], a);
        z = fmaf(f, sl[i], z);
      }
  }
  const float o = a / z;
  if (BF16)
    ((unsigned short*)p.out)[oi] = f32_to_bf16_bits(o);
  else
    ((float*)p.out)[oi] = o;
  if (t == 0) p.lse[(size_t)b * p.H + h] = (M + __builtin_log2f(z)) * kLn2;
}

template <int D, int G, bool BF16>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  // kv heads fastest: the waves dispatched together read whole cache positions
  decode_split_kernel<D, G, BF16><<<dim3(p.Hkv, p.n_split, p.B), 64, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<D, G, BF16><<<dim3(p.H, p.B), D, 0, s>>>(p);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
  switch (p.H / p.Hkv) {
    case 1: return launch_t<D, 1, BF16>(p, s);
    case 2: return launch_t<D, 2, BF16>(p, s);
    case 3: return launch_t<D, 3, BF16>(p, s);
    case 4: return launch_t<D, 4, BF16>(p, s);
    case 6: return launch_t<D, 6, BF16>(p, s);
    case 8: return launch_t<D, 8, BF16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Batch-1 prefill cache row -> n_rows decode rows: 16-byte vectors, grid-stride.
__global__ __launch_bounds__(256) void replicate_kernel(const u32x4* __restrict__ src, char* __restrict__ dst,
                                                        size_t nvec, int n_rows, size_t row_stride) {
  const size_t total = nvec * (size_t)n_rows;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / nvec, v = i - r * nvec;
    *(u32x4*)(dst + r * row_stride + v * 16) = src[v];
  }
}

// Chunk append: 16-byte vectors of k_new / v_new [B, Tq, Hkv, D] into cache
// slots n_b .. n_b + Tq - 1; rows whose slots do not fit write nothing.
__global__ __launch_bounds__(256) void cache_append_kernel(const u32x4* __restrict__ kn, const u32x4* __restrict__ vn,
                                                           u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                           const int32_t* __restrict__ lens, int B, int Tq,
                                                           int T_max, size_t vec_per_pos) {
  const size_t per_row = (size_t)Tq * vec_per_pos, total = per_row * B;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int b = (int)(i / per_row);
    const size_t r = i - (size_t)b * per_row;
    const int n = lens[b];
    if (n < 0 || n > T_max - Tq) continue;
    const size_t dst = ((size_t)b * T_max + n) * vec_per_pos + r;
    kc[dst] = kn[i];
    vc[dst] = vn[i];
  }
}

}  // namespace

hipError_t launch_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const int32_t* cache_seqlens, int B, int Tq, int Hkv, int D, int T_max,
                               size_t elem_bytes, hipStream_t s) {
  const size_t vec_per_pos = (size_t)Hkv * D * elem_bytes / 16;
  const size_t total = vec_per_pos * Tq * B;
  const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 8192);
  cache_append_kernel<<<blocks, 256, 0, s>>>((const u32x4*)k_new, (const u32x4*)v_new, (u32x4*)k_cache,
                                             (u32x4*)v_cache, cache_seqlens, B, Tq, T_max, vec_per_pos);
  return hipGetLastError();
}

hipError_t launch_replicate(const void* src, void* dst, size_t n_bytes, int n_rows, size_t row_stride, hipStream_t s) {
  const size_t nvec = n_bytes / 16;
  const size_t total = nvec * (size_t)n_rows;
  const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 8192);
  replicate_kernel<<<blocks, 256, 0, s>>>((const u32x4*)src, (char*)dst, nvec, n_rows, row_stride);
  return hipGetLastError();
}

bool decode_group_supported(int G) { return G == 1 || G == 2 || G == 3 || G == 4 || G == 6 || G == 8; }

hipError_t launch_decode(const DecodeParams& p, bool bf16, hipStream_t s) {
  switch (p.D) {
    case 32: return bf16 ? launch_g<32, true>(p, s) : launch_g<32, false>(p, s);
    case 64: return bf16 ? launch_g<64, true>(p, s) : launch_g<64, false>(p, s);
    case 128: return bf16 ? launch_g<128, true>(p, s) : launch_g<128, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
