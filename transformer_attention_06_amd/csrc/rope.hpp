// Per-lane pieces of the QK prologue (weightless RMSNorm, then half-split
// RoPE) for a head vector spread over D/8 lanes, 8 elements per lane ("nanochat
// Admin & Developer Guide", section 3: RMSNorm without weights and rotary
// embeddings with base 100000, rotating element d with element d + D/2).
// Shared by the prologue kernels and the decode step.
#pragma once

#include "common.hpp"

namespace nc {

// value of the lane holding the other half of the head vector (lane ^ HALF)
template <int HALF>
__device__ __forceinline__ float partner(float v) {
  if (HALF == 8) return dpp_mov<0x128>(v);  // whole 16-lane row: row_ror by 8
  return shfl_xor(v, HALF);
}

template <bool BF16>
__device__ __forceinline__ void ld8(const void* base, size_t off, float* f) {
  if (BF16) {
    unpack8_bf16(*(const u32x4*)((const unsigned short*)base + off), f);
  } else {
    const f32x4* p = (const f32x4*)((const float*)base + off);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void st8(void* base, size_t off, const float* f) {
  if (BF16) {
    *(u32x4*)((unsigned short*)base + off) = pack8_bf16(f);
  } else {
    f32x4* p = (f32x4*)((float*)base + off);
    p[0] = (f32x4){f[0], f[1], f[2], f[3]};
    p[1] = (f32x4){f[4], f[5], f[6], f[7]};
  }
}

// y = x * inv_r rotated by the angles whose cos/sin this lane holds: the low
// half of the vector takes y_d c - y_{d+D/2} s, the high half y_d s + y_{d+D/2} c.
template <int HALF>
__device__ __forceinline__ void rotate8(const float* x, float inv_r, const float* cs, const float* sn, bool low,
                                        float* res) {
  float y[8], yp[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e] * inv_r;
#pragma unroll
  for (int e = 0; e < 8; ++e) yp[e] = partner<HALF>(y[e]);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    res[e] = low ? fmaf(y[e], cs[e], -yp[e] * sn[e]) : fmaf(yp[e], sn[e], y[e] * cs[e]);
}

// cos/sin of the 8 angles of lane c (its pair index is c mod HALF) at position pos
template <int D>
__device__ __forceinline__ void load_angles8(const float* cos_tab, const float* sin_tab, int pos, int c, float* cs,
                                             float* sn) {
  constexpr int HALF = D / 16;
  const size_t toff = (size_t)pos * (D / 2) + (c % HALF) * 8;
  const f32x4* pc = (const f32x4*)(cos_tab + toff);
  const f32x4* ps = (const f32x4*)(sin_tab + toff);
  const f32x4 c0 = pc[0], c1 = pc[1], s0 = ps[0], s1 = ps[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cs[i] = c0[i];
    cs[4 + i] = c1[i];
    sn[i] = s0[i];
    sn[4 + i] = s1[i];
  }
}

// The prologue of one head vector: lane c of its D/8-lane group holds
// elements 8c .. 8c + 7 of x on entry and of RoPE(RMSNorm(x), pos) on return.
// Every lane of the group must be active.
template <int D>
__device__ __forceinline__ void prologue8(const float* x, const float* cs, const float* sn, int c, float eps,
                                          float* res) {
  constexpr int LPR = D / 8, HALF = LPR / 2;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  ss = group_sum<LPR>(ss);
  const float inv_r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
  rotate8<HALF>(x, inv_r, cs, sn, c < HALF, res);
}

}  // namespace nc
