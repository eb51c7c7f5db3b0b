// Attention forward for gfx950.
//
// Computes causal grouped-query attention with a sliding window, as used by
// nanochat ("nanochat Admin & Developer Guide", section 3 "Sliding-window
// attention" and section 6 "Attention: FA3 with SDPA Fallback"):
//   s_ij = scale <q_i, k_j> over keys i - w < j <= i,
//   lse_i = ln sum_j exp(s_ij),  out_i = sum_j exp(s_ij - lse_i) v_j.
//
// bf16 kernel (flash-style, one pass over the keys with an online softmax):
//   * workgroup = 128 queries of one (b, h); 4 waves, 32 queries each;
//   * K/V tiles of 64 keys staged in LDS, the next tile prefetched into
//     registers while the current one is consumed;
//   * S^T = K Q^T on 32x32x16 bf16 MFMA, so that each lane owns one query
//     column: the row max and row sum need no cross-lane reduction except
//     one exchange between the two half-waves;
//   * the exponentiated scores come straight out of the accumulator in the
//     B-operand layout of O^T += V^T P^T (the contraction index is permuted
//     identically on both operands), and V^T is read with LDS transpose
//     reads;
//   * tiles entirely outside the causal band or window are never visited;
//     element masks are applied only on tiles that cut the band's edges.
// f32 kernel: plain per-query loop in float32, for the fp32 configurations.

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace nc {
namespace {

constexpr int FWD_BM = 128;  // queries per workgroup
constexpr int FWD_BN = 64;   // keys per tile
constexpr int FWD_THREADS = 256;

template <int D>
__global__ __launch_bounds__(FWD_THREADS, 2) void attn_fwd_bf16_kernel(FwdParams p) {
  constexpr int LD = D + 8;  // LDS row stride (elements): 16-byte pad per row
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int LOADS = FWD_BN * CPR / FWD_THREADS;
  static_assert(LOADS >= 1 && FWD_BN * CPR % FWD_THREADS == 0, "tile/thread mismatch");
  __shared__ __attribute__((aligned(16))) unsigned short k_lds[FWD_BN * LD];
  __shared__ __attribute__((aligned(16))) unsigned short v_lds[FWD_BN * LD];

  const int T = p.T;
  const int nqt = (T + FWD_BM - 1) / FWD_BM;
  const int N = nqt * p.H * p.B;
  const int logical = xcd_remap(blockIdx.x, N);
  const int bh = logical / nqt;
  const int qt = nqt - 1 - (logical - bh * nqt);  // late (heavier) query tiles first
  const int b = bh / p.H, h = bh - b * p.H;
  const int g = h / (p.H / p.Hkv);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hh = lane >> 5;
  const int q0 = qt * FWD_BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + li;
  const bool q_valid = qi < T;

  const size_t qrs = (size_t)p.H * D;
  const size_t kvrs = (size_t)p.Hkv * D;
  const unsigned short* qp = (const unsigned short*)p.q + (size_t)b * T * qrs + (size_t)h * D;
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)b * T * kvrs + (size_t)g * D;
  const unsigned short* vp = (const unsigned short*)p.v + (size_t)b * T * kvrs + (size_t)g * D;

  // Q as the B operand of S^T = K Q^T: lane (li, hh) holds q[qi][16 s + 8 hh + e].
  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (q_valid) w = *(const u32x4*)(qp + (size_t)qi * qrs + 16 * s + 8 * hh);
    qf[s] = __builtin_bit_cast(bf16x8, w);
  }

  const bool full = p.window <= 0;
  const int win = p.window;
  const int kv_hi = min(T - 1, q0 + FWD_BM - 1);
  const int kv_lo = full ? 0 : max(0, q0 - win + 1);
  const int t_begin = kv_lo / FWD_BN, t_end = kv_hi / FWD_BN;

  float m2 = -INFINITY;  // running max of scale*log2(e)*s for this query
  float lsum = 0.f;      // running sum over this lane's half of the keys
  f32x16 o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = (f32x16){};

  u32x4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int jt) {
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int c = tid + n * FWD_THREADS;
      const int row = c / CPR, ch = c - row * CPR;
      const int j = jt * FWD_BN + row;
      if (j < T) {
        kreg[n] = *(const u32x4*)(kp + (size_t)j * kvrs + ch * 8);
        vreg[n] = *(const u32x4*)(vp + (size_t)j * kvrs + ch * 8);
      } else {
        kreg[n] = (u32x4){0u, 0u, 0u, 0u};
        vreg[n] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int c = tid + n * FWD_THREADS;
      const int row = c / CPR, ch = c - row * CPR;
      *(u32x4*)(k_lds + row * LD + ch * 8) = kreg[n];
      *(u32x4*)(v_lds + row * LD + ch * 8) = vreg[n];
    }
  };

  const int grp = lane >> 4, t16 = lane & 15;
  // per-lane offset of the transpose read of V^T (rows 4 hh + t16/4, columns 16 (grp&1) + 4 (t16&3))
  const int vtr_off = (4 * hh + (t16 >> 2)) * LD + 16 * (grp & 1) + 4 * (t16 & 3);

  load_tile(t_begin);
  for (int jt = t_begin; jt <= t_end; ++jt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (jt < t_end) load_tile(jt + 1);

    const int j0 = jt * FWD_BN;
    const bool any = (j0 <= qw + 31) && (full || j0 + FWD_BN - 1 > qw - win);
    if (!any) continue;
    const bool interior = (j0 + FWD_BN - 1 <= qw) && (full || j0 > qw + 31 - win);

    f32x16 s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      s[jb] = (f32x16){};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const bf16x8 a = *(const bf16x8*)(k_lds + (jb * 32 + li) * LD + 16 * st + 8 * hh);
        s[jb] = mfma32(a, qf[st], s[jb]);
      }
    }
    // s[jb][r] = S[key j0 + 32 jb + 8 (r/4) + 4 hh + r%4][query qi]
    if (!interior) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * jb + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool vis = (j <= qi) && (full || j > qi - win);
          if (!vis) s[jb][r] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[jb][r]);
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m2, mx * p.scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2_fast(m2 - m_use);
    m2 = m_new;

    float pv[2][16];
    float rs = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[jb][r] = exp2_fast(fmaf(s[jb][r], p.scale_log2, -m_use));
        rs += pv[jb][r];
      }
    lsum = fmaf(lsum, alpha, rs);
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] *= alpha;

#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pb = to_bf16x8(&pv[jb][8 * u]);
        const unsigned short* vb = v_lds + (32 * jb + 16 * u) * LD + vtr_off;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const s16x4 x1 = lds_read_tr16(vb + 32 * d);
          const s16x4 x2 = lds_read_tr16(vb + 32 * d + 8 * LD);
          o[d] = mfma32(cat_bf16x8(x1, x2), pb, o[d]);
        }
      }
  }

  const float lt = lsum + shfl_xor(lsum, 32);
  if (q_valid) {
    const float inv = 1.f / lt;
    unsigned short* op = (unsigned short*)p.out + ((size_t)b * T + qi) * qrs + (size_t)h * D;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 w;
        w[0] = pack2_bf16(o[d][4 * rg] * inv, o[d][4 * rg + 1] * inv);
        w[1] = pack2_bf16(o[d][4 * rg + 2] * inv, o[d][4 * rg + 3] * inv);
        *(u32x2*)(op + 32 * d + 8 * rg + 4 * hh) = w;
      }
    if (hh == 0) p.lse[((size_t)b * p.H + h) * T + qi] = (m2 + __builtin_log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// float32: one thread per query, online softmax over its visible keys.
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(FwdParams p) {
  const int T = p.T;
  const int qi = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (qi >= T) return;
  const int g = h / (p.H / p.Hkv);
  const float* q = (const float*)p.q + (((size_t)b * T + qi) * p.H + h) * D;
  const float* kb = (const float*)p.k + ((size_t)b * T * p.Hkv + g) * D;
  const float* vb = (const float*)p.v + ((size_t)b * T * p.Hkv + g) * D;
  const size_t rs = (size_t)p.Hkv * D;
  float qr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = q[d];
    acc[d] = 0.f;
  }
  const int lo = p.window <= 0 ? 0 : max(0, qi - p.window + 1);
  float m = -INFINITY, l = 0.f;
  for (int j = lo; j <= qi; ++j) {
    const float* kr = kb + (size_t)j * rs;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qr[d], kr[d], s);
    s *= p.scale;
    const float mn = fmaxf(m, s);
    const float a = expf(m - mn);
    const float e = expf(s - mn);
    l = l * a + e;
    const float* vr = vb + (size_t)j * rs;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], a, e * vr[d]);
    m = mn;
  }
  float* o = (float*)p.out + (((size_t)b * T + qi) * p.H + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = acc[d] * inv;
  p.lse[((size_t)b * p.H + h) * T + qi] = m + logf(l);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdParams& p, hipStream_t s) {
  const int nqt = (p.T + FWD_BM - 1) / FWD_BM;
  const dim3 grid(nqt * p.H * p.B), block(FWD_THREADS);
  switch (p.D) {
    case 32: attn_fwd_bf16_kernel<32><<<grid, block, 0, s>>>(p); break;
    case 64: attn_fwd_bf16_kernel<64><<<grid, block, 0, s>>>(p); break;
    case 128: attn_fwd_bf16_kernel<128><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const FwdParams& p, hipStream_t s) {
  const dim3 grid((p.T + 63) / 64, p.H, p.B), block(64);
  switch (p.D) {
    case 32: attn_fwd_f32_kernel<32><<<grid, block, 0, s>>>(p); break;
    case 64: attn_fwd_f32_kernel<64><<<grid, block, 0, s>>>(p); break;
    case 128: attn_fwd_f32_kernel<128><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nc
