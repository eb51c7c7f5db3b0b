// Single-token KV-cache decode for gfx950 (split-K over ragged lengths).
//
// Row b holds L_b = seqlens[b] cached keys including the current token; its
// query sits at position L_b - 1 and attends to cache positions
// max(0, L_b - w) .. L_b - 1 (all of them for a full-context layer).
// ("nanochat Admin & Developer Guide", section 7 "KV cache": per-layer
// (B, T, H, D) cache, per-row int32 lengths; section 6: single-token decode
// slices the key window.)
//
// decode_split: one workgroup per (split of 256 cache positions, kv head,
//   row). Each group of D/8 lanes streams one cache row at a time (D/8 lanes
//   x 16 bytes = the contiguous head vector), so a wave reads whole 256-byte
//   rows; the dot product is finished with a butterfly of cross-lane
//   exchanges inside the group. Each group keeps an online softmax
//   (m, l, acc) per query head of the GQA group; the groups are merged in
//   LDS and one partial per (row, head, split) goes to the workspace.
//   Splits outside a row's key range exit without reading anything.
// decode_combine: merges a row's partials into out and lse. A length
//   outside 1..T_max yields NaN out and lse for that row.

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace nc {
namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_KU = 4;  // cache rows in flight per group

template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t elem_off, float* f) {
  if (BF16) {
    unpack8_bf16(__builtin_nontemporal_load((const u32x4*)((const unsigned short*)base + elem_off)), f);
  } else {
    const f32x4* p = (const f32x4*)((const float*)base + elem_off);
    const f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  }
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(DEC_THREADS) void decode_split_kernel(DecodeParams p) {
  constexpr int LPR = D / 8;               // lanes per cache row
  constexpr int NG = DEC_THREADS / LPR;    // row groups per workgroup
  __shared__ float red_acc[NG * D];
  __shared__ float red_m[NG], red_l[NG];

  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = p.seqlens[b];
  if (L < 1 || L > p.T_max) return;
  const bool full = p.window <= 0 || p.window >= L;
  const int lo = full ? 0 : L - p.window;
  const int k_begin = max(lo, sp * kDecodeSplit);
  const int k_end = min(L, (sp + 1) * kDecodeSplit);  // exclusive
  if (k_begin >= k_end) return;

  const int tid = threadIdx.x;
  const int grp = tid / LPR, c = tid - (tid / LPR) * LPR;
  const int H = p.H;
  const size_t rs = (size_t)p.Hkv * D;  // elements per cache position
  const size_t cache_base = (size_t)b * p.T_max * rs + (size_t)g * D + c * 8;

  float qf[G][8];
#pragma unroll
  for (int hq = 0; hq < G; ++hq) {
    float t[8];
    if (BF16)
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
    for (int e = 0; e < 8; ++e) qf[hq][e] = t[e] * p.scale_log2;
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int hq = 0; hq < G; ++hq) {
    m[hq] = -INFINITY;
    l[hq] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hq][e] = 0.f;
  }

  for (int j = k_begin + grp; j < k_end; j += NG * DEC_KU) {
    float kr[DEC_KU][8], vr[DEC_KU][8];
#pragma unroll
    for (int u = 0; u < DEC_KU; ++u) {
      const int jj = j + u * NG;
      if (jj < k_end) {
        load8<BF16>(p.k_cache, cache_base + (size_t)jj * rs, kr[u]);
        load8<BF16>(p.v_cache, cache_base + (size_t)jj * rs, vr[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < DEC_KU; ++u) {
      const int jj = j + u * NG;
      if (jj >= k_end) break;  // uniform across the group
#pragma unroll
      for (int hq = 0; hq < G; ++hq) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(qf[hq][e], kr[u][e], s);
#pragma unroll
        for (int msk = LPR / 2; msk >= 1; msk >>= 1) s += shfl_xor(s, msk);
        const float mn = fmaxf(m[hq], s);
        const float a = exp2_fast(m[hq] - mn);
        const float pe = exp2_fast(s - mn);
        l[hq] = fmaf(l[hq], a, pe);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hq][e] = fmaf(acc[hq][e], a, pe * vr[u][e]);
        m[hq] = mn;
      }
    }
  }

  // merge the groups, one query head at a time
  float* part_row = p.part + (((size_t)b * H + g * G) * p.n_split + sp) * (D + 2);
#pragma unroll
  for (int hq = 0; hq < G; ++hq) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) red_acc[grp * D + c * 8 + e] = acc[hq][e];
    if (c == 0) {
      red_m[grp] = m[hq];
      red_l[grp] = l[hq];
    }
    __syncthreads();
    if (tid < D) {
      float M = -INFINITY;
      for (int r = 0; r < NG; ++r) M = fmaxf(M, red_m[r]);
      float a = 0.f, z = 0.f;
      for (int r = 0; r < NG; ++r) {
        const float f = red_m[r] == -INFINITY ? 0.f : exp2_fast(red_m[r] - M);
        a = fmaf(f, red_acc[r * D + tid], a);
        z = fmaf(f, red_l[r], z);
      }
      float* dst = part_row + (size_t)hq * p.n_split * (D + 2);
      dst[tid] = a;
      if (tid == 0) {
        dst[D] = M;
        dst[D + 1] = z;
      }
    }
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeParams p) {
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int L = p.seqlens[b];
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
  const int s0 = lo / kDecodeSplit, s1 = (L - 1) / kDecodeSplit;
  const float* part = p.part + ((size_t)b * p.H + h) * p.n_split * (D + 2);
  float M = -INFINITY;
  for (int s = s0; s <= s1; ++s) M = fmaxf(M, part[(size_t)s * (D + 2) + D]);
  float a = 0.f, z = 0.f;
  for (int s = s0; s <= s1; ++s) {
    const float* ps = part + (size_t)s * (D + 2);
    const float f = exp2_fast(ps[D] - M);
    a = fmaf(f, ps[t], a);
    z = fmaf(f, ps[D + 1], z);
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
  decode_split_kernel<D, G, BF16><<<dim3(p.n_split, p.Hkv, p.B), DEC_THREADS, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_combine_kernel<D, BF16><<<dim3(p.H, p.B), D, 0, s>>>(p);
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

}  // namespace

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
