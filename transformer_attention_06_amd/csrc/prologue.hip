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


#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "rope.hpp"

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

}  // namespace

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
