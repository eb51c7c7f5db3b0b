// QK prologue for gfx950: weightless RMSNorm followed by half-split RoPE,
// and its backward; plus the RoPE cos/sin table.
//
// ("nanochat Admin & Developer Guide", section 3: rotary embeddings with
// base theta 100000 and a table computed past the sequence length; queries
// and keys RMS-normalised with no learnable parameters. "nanochat (Fucina
// port)", "Architecture": no-weight RMSNorm, half-split RoPE from an
// inverse-frequency table.)
//
// Forward, per head vector x of length D at position p:
//   y = x / sqrt(mean(x^2) + eps);
//   for d < D/2: (y_d, y_{d+D/2}) <- (y_d c - y_{d+D/2} s, y_d s + y_{d+D/2} c)
//   with c = cos(p * base^(-2d/D)), s = sin(...).
// Backward: u = R(-theta) dy, r = sqrt(mean(x^2) + eps),
//   dx = u / r - x <x, u> / (D r^3).
// One group of D/8 lanes per head vector (16 bytes of bf16 per lane); the
// sums of squares and the pairing of d with d + D/2 are cross-lane
// exchanges inside the group. Statistics in float32.
//
// Decode append (the step before single-token decode, in the manner of the
// in-place cache update of FA3's kvcache call that the pages describe:
// section 7 "KV cache", per-row int32 cache_seqlens): row b holds
// n = cache_seqlens[b] cached tokens; the new token sits at position n. Its
// q and k get the forward prologue at position n, q' goes to a float32
// buffer (it is never stored in the model's dtype), k'
// and the new v are written into cache position n, and the row's key count
// n + 1 is stored for the decode kernels. A row whose n is outside
// 0 .. min(T_max, T_rope) - 1 writes nothing into the cache and gets key
// count 0 (the decode then yields NaN for it).

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace nc {
namespace {

__global__ void rope_table_kernel(int T_rope, int half, double base, float* __restrict__ c,
                                  float* __restrict__ s) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)T_rope * half) return;
  const int pos = (int)(i / half), d = (int)(i - (long)(i / half) * half);
  const double inv = pow(base, -2.0 * d / (2.0 * half));
  const double th = (double)pos * inv;
  double sn, cs;
  sincos(th, &sn, &cs);
  c[i] = (float)cs;
  s[i] = (float)sn;
}

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

template <int D, bool BF16, bool BWD>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueParams p) {
  constexpr int LPR = D / 8;
  constexpr int HALF = LPR / 2;  // partner lane distance
  const long nq = (long)p.B * p.T * p.H;
  const long nrows = nq + (long)p.B * p.T * p.Hkv;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = gid / LPR;
  const int c = (int)(gid - row * LPR);
  const bool valid = row < nrows;
  const long rr = valid ? row : 0;

  // which tensor and which (b, t)
  const bool is_q = rr < nq;
  const long r2 = is_q ? rr : rr - nq;
  const int heads = is_q ? p.H : p.Hkv;
  const long bt = r2 / heads;
  const int b = (int)(bt / p.T), t = (int)(bt - (long)(bt / p.T) * p.T);
  const size_t off = (size_t)r2 * D + c * 8;
  const void* xin = is_q ? p.q : p.k;

  int pos = t + (p.pos_offset ? p.pos_offset[b] : 0);
  const bool pos_ok = pos >= 0 && pos < p.T_rope;
  if (!pos_ok) pos = 0;

  float x[8], dy[8];
  ld8<BF16>(xin, off, x);
  if (BWD) ld8<BF16>(is_q ? p.dq_out : p.dk_out, off, dy);

  float cs[8], sn[8];
  load_angles8<D>(p.cos_tab, p.sin_tab, pos, c, cs, sn);
  const bool low = c < HALF;

  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  ss = group_sum<LPR>(ss);
  const float r = sqrtf(ss * (1.0f / D) + p.eps);
  const float inv_r = 1.0f / r;

  float res[8];
  if (!BWD) {
    rotate8<HALF>(x, inv_r, cs, sn, low, res);
  } else {
    // u = R(-theta) dy: low half a' = a c + b s, high half b' = -a s + b c
    float dp[8], u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dp[e] = partner<HALF>(dy[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      u[e] = low ? fmaf(dy[e], cs[e], dp[e] * sn[e]) : fmaf(dy[e], cs[e], -dp[e] * sn[e]);
    float xu = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) xu = fmaf(x[e], u[e], xu);
    xu = group_sum<LPR>(xu);
    const float k3 = xu * inv_r * inv_r * inv_r * (1.0f / D);
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] = fmaf(u[e], inv_r, -x[e] * k3);
  }
  if (!pos_ok) {
#pragma unroll
    for (int e = 0; e < 8; ++e) res[e] = NAN;
  }
  if (valid) st8<BF16>(is_q ? p.q_out : p.k_out, off, res);
}

template <int D>
hipError_t launch_d(const PrologueParams& p, bool bf16, bool bwd, hipStream_t s) {
  const long rows = (long)p.B * p.T * (p.H + p.Hkv);
  const long threads = rows * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (bf16) {
    if (bwd)
      prologue_kernel<D, true, true><<<blocks, 256, 0, s>>>(p);
    else
      prologue_kernel<D, true, false><<<blocks, 256, 0, s>>>(p);
  } else {
    if (bwd)
      prologue_kernel<D, false, true><<<blocks, 256, 0, s>>>(p);
    else
      prologue_kernel<D, false, false><<<blocks, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

// Rows: B*H query vectors, then B*Hkv new keys, then B*Hkv new values; one
// group of D/8 lanes per row. Every lane runs the group exchanges (rows never
// straddle a group); only the stores are predicated.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void decode_append_kernel(AppendParams p) {
  constexpr int LPR = D / 8;
  constexpr int HALF = LPR / 2;
  const long nq = (long)p.B * p.H, nk = (long)p.B * p.Hkv;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = gid / LPR;
  const int c = (int)(gid - row * LPR);
  const bool valid = row < nq + 2 * nk;
  const long rr = valid ? row : 0;
  const int kind = rr < nq ? 0 : (rr < nq + nk ? 1 : 2);  // q, k, v
  const long r2 = kind == 0 ? rr : rr - nq - (kind == 2 ? nk : 0);
  const int heads = kind == 0 ? p.H : p.Hkv;
  const int b = (int)(r2 / heads), hd = (int)(r2 - (long)b * heads);
  const int n = p.cache_seqlens[b];
  const bool ok = n >= 0 && n < p.T_max && n < p.T_rope;
  const int pos = ok ? n : 0;

  const void* src = kind == 0 ? p.q : (kind == 1 ? p.k_new : p.v_new);
  float x[8];
  ld8<BF16>(src, (size_t)r2 * D + c * 8, x);
  float cs[8], sn[8];
  load_angles8<D>(p.cos_tab, p.sin_tab, pos, c, cs, sn);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  ss = group_sum<LPR>(ss);
  const float inv_r = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
  float res[8];
  rotate8<HALF>(x, inv_r, cs, sn, c < HALF, res);
  if (!valid) return;
  if (kind == 0) {
    st8<false>(p.q_out, (size_t)r2 * D + c * 8, res);  // q' stays float32
    if (hd == 0 && c == 0) p.seqlens_out[b] = ok ? n + 1 : 0;
  } else if (ok) {
    const size_t dst = (((size_t)b * p.T_max + n) * p.Hkv + hd) * D + c * 8;
    st8<BF16>(kind == 1 ? p.k_cache : p.v_cache, dst, kind == 1 ? res : x);
  }
}

template <int D>
hipError_t launch_append_d(const AppendParams& p, bool bf16, hipStream_t s) {
  const long threads = ((long)p.B * p.H + 2L * p.B * p.Hkv) * (D / 8);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (bf16)
    decode_append_kernel<D, true><<<blocks, 256, 0, s>>>(p);
  else
    decode_append_kernel<D, false><<<blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_append(const AppendParams& p, bool bf16, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_append_d<32>(p, bf16, s);
    case 64: return launch_append_d<64>(p, bf16, s);
    case 128: return launch_append_d<128>(p, bf16, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rope_table(int T_rope, int D, double base, float* c, float* sn, hipStream_t s) {
  const long n = (long)T_rope * (D / 2);
  rope_table_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(T_rope, D / 2, base, c, sn);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueParams& p, bool bf16, bool backward, hipStream_t s) {
  switch (p.D) {
    case 32: return launch_d<32>(p, bf16, backward, s);
    case 64: return launch_d<64>(p, bf16, backward, s);
    case 128: return launch_d<128>(p, bf16, backward, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
