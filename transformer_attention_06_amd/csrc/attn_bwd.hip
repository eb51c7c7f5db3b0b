// Attention backward for gfx950.
//
// Gradients of L = sum(out * dout) for the causal sliding-window GQA
// attention of attn_fwd.hip, with the probabilities recomputed from the
// saved log-sum-exp instead of stored:
//   P_ij = exp(s_ij - lse_i), dP_ij = <dout_i, v_j>, delta_i = <dout_i, out_i>,
//   dS_ij = P_ij (dP_ij - delta_i),
//   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_{h in group} sum_i dS_ij q_i,
//   dv_j = sum_{h in group} sum_i P_ij dout_i.
// (The pages only say upstream differentiates attention with autograd and
// that the .NET port hand-writes its backward kernels — "nanochat (Python)"
// and "NanoChat.NET" catalog pages, "Model & kernels"; the formulas are the
// plain chain rule through the softmax.)
//
// bf16 path, two kernels, no atomics:
//   dq:   one workgroup per (b, h, 128-query tile), the forward kernel's
//         structure: q and dO stay in registers as B operands, K/V tiles of
//         64 keys stream through double-buffered LDS, S^T = K Q^T and
//         dP^T = V dO^T give one query column per lane, dS is formed from
//         the row statistics, and dQ^T += K^T dS^T takes K^T from LDS
//         transpose reads. S and dP are recomputed here rather than
//         exchanged with dkdv, which keeps dQ free of float atomics. It
//         forms the row statistics delta_i = <dout_i, out_i> and
//         lse_i * log2(e) itself and stores them for dkdv.
//   dkdv: one workgroup per (b, kv head, 64-key tile), two per CU; each of
//         its 4 waves keeps 16 keys' K and V fragments in registers and
//         accumulates dK^T and dV^T for them over every query head of the
//         GQA group and every 64-query tile that intersects the band, on
//         16x16x32 MFMA. S = Q K^T and dP = dO V^T come out with one key
//         column per lane, which is directly the B-operand layout of
//         dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T are LDS transpose
//         reads. Q/dO tiles and the per-row statistics stream into LDS with
//         buffer-to-LDS loads running NBUF - 1 steps ahead; LDS addresses are
//         per-lane constants.
// f32 path: row statistics, then plain per-query (dq) and per-key (dk, dv)
// loops in float32.

#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace nc {
namespace {

constexpr int BWD_THREADS = 256;
constexpr int NBUF = 2;  // q/dO tile buffers: loads run one step ahead
constexpr int DQ_BM = 128;  // queries per dq workgroup (32 per wave)
constexpr int DQ_BN = 64;   // keys per dq tile

// --------------------------------------------------------------------------
// Stores one head-vector gradient held in MFMA result layout: lane (li, hh)
// holds g[db][4 rg + e] = dy[32 db + 8 rg + 4 hh + e] / mul, the lane with
// the other hh the rest of the vector. Without the prologue the stored
// values are dy; with it, the gradient w.r.t. the raw vector x at position
// pos ("nanochat Admin & Developer Guide", section 3: weightless RMSNorm,
// then half-split RoPE):
//   u = R(-theta) dy,  r = sqrt(mean(x^2) + eps),  dx = u / r - x <x, u> / (D r^3).
// All 64 lanes must call it (the row sums pair lanes l and l ^ 32); valid
// says whether this lane's vector exists. xw holds the lane's part of x as
// loaded by load_row_words (nullptr: no prologue).
template <int D>
__device__ __forceinline__ void load_row_words(const unsigned short* xrow, bool valid, int hh, u32x2* xw) {
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      xw[4 * d + rg] = valid ? *(const u32x2*)(xrow + 32 * d + 8 * rg + 4 * hh) : (u32x2){0u, 0u};
}
template <int D>
__device__ __forceinline__ void store_grad_row(const BwdParams& p, const f32x16* g, float mul, bool valid,
                                               const u32x2* xw, int pos, int hh, unsigned short* orow) {
  constexpr int ND = D / 32;
  if (!xw) {
    if (valid) {
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          u32x2 w;
          w[0] = pk_bf16(g[d][4 * rg] * mul, g[d][4 * rg + 1] * mul);
          w[1] = pk_bf16(g[d][4 * rg + 2] * mul, g[d][4 * rg + 3] * mul);
          *(u32x2*)(orow + 32 * d + 8 * rg + 4 * hh) = w;
        }
    }
    return;
  }
  const bool pos_ok = pos >= 0 && pos < p.T_rope;
  const int tp = (valid && pos_ok) ? pos : 0;
  float x[ND][16], u[ND][16];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const u32x2 w = xw[4 * d + rg];
      x[d][4 * rg + 0] = __builtin_bit_cast(float, w[0] << 16);
      x[d][4 * rg + 1] = __builtin_bit_cast(float, w[0] & 0xffff0000u);
      x[d][4 * rg + 2] = __builtin_bit_cast(float, w[1] << 16);
      x[d][4 * rg + 3] = __builtin_bit_cast(float, w[1] & 0xffff0000u);
    }
  // u = R(-theta) dy over the pairs (i, i + D/2): low a' = a c + b s, high b' = -a s + b c
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const bool low = ND >= 2 ? d < ND / 2 : rg < 2;
      if (!low) continue;
      const int pd = ND >= 2 ? d + ND / 2 : d, prg = ND >= 2 ? rg : rg + 2;
      const int i = 32 * d + 8 * rg + 4 * hh;  // < D/2
      const f32x4 c4 = *(const f32x4*)(p.cos_tab + (size_t)tp * (D / 2) + i);
      const f32x4 s4 = *(const f32x4*)(p.sin_tab + (size_t)tp * (D / 2) + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = g[d][4 * rg + e] * mul, b = g[pd][4 * prg + e] * mul;
        u[d][4 * rg + e] = fmaf(a, c4[e], b * s4[e]);
        u[pd][4 * prg + e] = fmaf(b, c4[e], -a * s4[e]);
      }
    }
  float ss = 0.f, xu = 0.f;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      ss = fmaf(x[d][e], x[d][e], ss);
      xu = fmaf(x[d][e], u[d][e], xu);
    }
  ss = sum_mod<32>(ss);
  xu = sum_mod<32>(xu);
  const float inv_r = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
  const float k3 = xu * inv_r * inv_r * inv_r * (1.0f / D);
  if (valid) {
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pos_ok ? fmaf(u[d][4 * rg + e], inv_r, -x[d][4 * rg + e] * k3) : NAN;
        *(u32x2*)(orow + 32 * d + 8 * rg + 4 * hh) = (u32x2){pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3])};
      }
  }
}

// --------------------------------------------------------------------------
// float32 path: delta = rowsum(dout * out), lse2 = lse * log2(e).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(BwdParams p) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long rows = (long)p.B * p.T * p.H;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = gid / LPR;
  const int c = (int)(gid - row * LPR);
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + c * 8;
    const f32x4* pa = (const f32x4*)((const float*)p.dout + off);
    const f32x4* po = (const f32x4*)((const float*)p.out + off);
    const f32x4 a0 = pa[0], a1 = pa[1], o0 = po[0], o1 = po[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(a1[i], o1[i], fmaf(a0[i], o0[i], acc));
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += shfl_xor(acc, m);
  if (row < rows && c == 0) {
    // row = (b * T + t) * H + h  ->  [b, h, t]
    const long bt = row / p.H;
    const int h = (int)(row - bt * p.H);
    const long b = bt / p.T;
    const int t = (int)(bt - b * p.T);
    const size_t o = ((size_t)b * p.H + h) * p.T + t;
    p.delta[o] = acc;
    p.lse2[o] = p.lse[o] * kLog2e;
  }
}

// --------------------------------------------------------------------------
// dK and dV: one workgroup per (b, kv head, 64-key tile), 4 waves of 16 keys,
// two workgroups per CU, 16x16x32 bf16 MFMA, 64-query steps. With 16 keys a
// wave's stationary registers (K, V fragments and the dK, dV accumulators)
// leave room for two waves of independent workgroups on every SIMD, which
// hide each other's LDS and arithmetic latency (with 32 keys per wave on
// 32x32x16 MFMA only one wave fits per SIMD). Layouts (lane l,
// t = l % 16, g = l / 16): A operands hold A[t][8 g + e], B operands
// B[8 g + e][t], results C[4 g + r][t].
//   S = Q K^T per 16-query block: A = q rows (LDS), B = K^T (registers),
//     result: one key column per lane, queries 4 g + r of the block;
//   dV^T += dO^T P and dK^T += Q^T dS per 16-wide block of d over 32 queries:
//     A = dO^T / Q^T from transpose reads of rows {4 g .. 4 g + 3} and
//     {16 + 4 g .. 16 + 4 g + 3}, B = P / dS of the lane's key for exactly
//     those queries (the two 16-query blocks of S), so the contraction index
//     is paired identically on both operands.
constexpr int K16_WAVES = 4;               // waves per workgroup (two workgroups per CU)
constexpr int K16_BN = 16 * K16_WAVES;     // keys per workgroup
constexpr int K16_BM = 64;                 // queries per step
constexpr int BWD16_THREADS = 64 * K16_WAVES;

// Stores one head-vector gradient held in the 16x16 result layout: lane
// (t, g) holds gr[db][r] = dy[16 db + 4 g + r] / mul; the lanes with the same
// t hold the rest. Prologue backward as in store_grad_row. All 64 lanes must
// call it; xw holds x[16 db + 4 g .. + 3] (nullptr: no prologue).
template <int D>
__device__ __forceinline__ void store_grad_row16(const BwdParams& p, const f32x4* gr, float mul, bool valid,
                                                 const u32x2* xw, int pos, int grp, unsigned short* orow) {
  constexpr int NB = D / 16;
  if (!xw) {
    if (valid) {
#pragma unroll
      for (int db = 0; db < NB; ++db)
        *(u32x2*)(orow + 16 * db + 4 * grp) =
            (u32x2){pk_bf16(gr[db][0] * mul, gr[db][1] * mul), pk_bf16(gr[db][2] * mul, gr[db][3] * mul)};
    }
    return;
  }
  const bool pos_ok = pos >= 0 && pos < p.T_rope;
  const int tp = (valid && pos_ok) ? pos : 0;
  float x[NB][4], u[NB][4];
#pragma unroll
  for (int db = 0; db < NB; ++db) {
    x[db][0] = __builtin_bit_cast(float, xw[db][0] << 16);
    x[db][1] = __builtin_bit_cast(float, xw[db][0] & 0xffff0000u);
    x[db][2] = __builtin_bit_cast(float, xw[db][1] << 16);
    x[db][3] = __builtin_bit_cast(float, xw[db][1] & 0xffff0000u);
  }
  // u = R(-theta) dy over the pairs (i, i + D/2): block db < NB/2 pairs with db + NB/2
#pragma unroll
  for (int db = 0; db < NB / 2; ++db) {
    const int i = 16 * db + 4 * grp;  // < D/2
    const f32x4 c4 = *(const f32x4*)(p.cos_tab + (size_t)tp * (D / 2) + i);
    const f32x4 s4 = *(const f32x4*)(p.sin_tab + (size_t)tp * (D / 2) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = gr[db][e] * mul, b = gr[db + NB / 2][e] * mul;
      u[db][e] = fmaf(a, c4[e], b * s4[e]);
      u[db + NB / 2][e] = fmaf(b, c4[e], -a * s4[e]);
    }
  }
  float ss = 0.f, xu = 0.f;
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss = fmaf(x[db][e], x[db][e], ss);
      xu = fmaf(x[db][e], u[db][e], xu);
    }
  ss = sum_mod<16>(ss);
  xu = sum_mod<16>(xu);
  const float inv_r = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
  const float k3 = xu * inv_r * inv_r * inv_r * (1.0f / D);
  if (valid) {
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pos_ok ? fmaf(u[db][e], inv_r, -x[db][e] * k3) : NAN;
      *(u32x2*)(orow + 16 * db + 4 * grp) = (u32x2){pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3])};
    }
  }
}

template <int D, bool PAIRED>
__global__ __launch_bounds__(BWD16_THREADS, 2) void attn_bwd_dkdv16_kernel(BwdParams p) {
  constexpr int NC = D / 8;   // chunks per row of the q/dO tiles (swizzled)
  constexpr int NK = D / 32;  // k-steps of S and dP
  constexpr int NB = D / 16;  // 16-wide blocks of d in dK^T, dV^T
  constexpr int NW = K16_WAVES;
  constexpr int BN = K16_BN, BM = K16_BM;
  constexpr int QT = BM * D;
  constexpr int RPI = 64 / NC;
  constexpr int QIPW = BM / RPI / NW;  // copy instructions per wave per tensor
  static_assert(QIPW >= 1 && BN == 16 * NW && BM == 64, "tile/wave mismatch");
  __shared__ __attribute__((aligned(16))) unsigned short q_lds[NBUF][QT];
  __shared__ __attribute__((aligned(16))) unsigned short do_lds[NBUF][QT];
  __shared__ __attribute__((aligned(16))) float lse2_lds[NBUF][BM];
  __shared__ __attribute__((aligned(16))) float dl_lds[NBUF][BM];

  const int T = p.T;
  const int nkt = (T + BN - 1) / BN;
  const int nunit = PAIRED ? (nkt + 1) / 2 : nkt;
  const int N = nunit * p.Hkv * p.B;
  const int logical = xcd_remap(blockIdx.x, N);
  const int bg = logical / nunit;
  const int r_pair = logical - bg * nunit;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int G = p.H / p.Hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int grp = lane >> 4, t16 = lane & 15;

  const unsigned qrs = (unsigned)(p.H * D);
  const unsigned kvrs = (unsigned)(p.Hkv * D);
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)b * T * kvrs + (size_t)g * D;
  const unsigned short* vp = (const unsigned short*)p.v + (size_t)b * T * kvrs + (size_t)g * D;

  const bool full = p.window <= 0;
  const int win = p.window;
  const unsigned wlim = full ? 0x80000000u : (unsigned)win;

  // ---- per-lane constant LDS offsets (the tiles use the swz_kv
  // permutation, which depends on row % 16, so +16 rows and +32 rows are
  // plain element offsets) ----
  // q/dO operand rows t (+16 qb + 32 ib) at column 32 ks + 8 g
  int aoff[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) aoff[ks] = swz_kv_off<NC>(t16, 32 * ks + 8 * grp);
  // transpose reads of dO^T / Q^T: rows 4 g + t/4 (+16) (+32 ib), columns 16 db + 4 (t % 4)
  int toff[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) toff[db] = swz_kv_off<NC>(4 * grp + (t16 >> 2), 16 * db + 4 * (t16 & 3));

  // ---- q/dO tile and row-statistics copies (buffer -> LDS) ----
  unsigned ld_off[QIPW];
  int ld_row[QIPW], ld_ch[QIPW];
#pragma unroll
  for (int n = 0; n < QIPW; ++n) {
    const int row = (wave * QIPW + n) * RPI + lane / NC;
    ld_row[n] = row;
    ld_ch[n] = (lane % NC) ^ (swz_kv<NC>(row) & (NC - 1));
    ld_off[n] = (unsigned)(row * qrs + ld_ch[n] * 8) * 2u;
  }
  const unsigned qspan = (unsigned)(((size_t)(T - 1) * qrs + D) * 2);
  auto run = [&](int kt) __attribute__((always_inline)) {
    const int j0 = kt * BN;
    const int kw = j0 + wave * 16;
    const int kj = kw + t16;  // this lane's key
    const size_t krow = ((size_t)b * T + kj) * kvrs + (size_t)g * D;  // its row of k, dk, dv
    u32x2 xk[NB];  // its raw k row (prologue backward), loaded during the last step
    const int i_last = full ? T - 1 : min(T - 1, j0 + BN - 1 + win - 1);
    const int it_begin = j0 / BM, n_it = i_last / BM - it_begin + 1;
    const int n_steps = G * n_it;
    // K and V fragments of this lane's key as B operands: x[kj][32 ks + 8 g + e]
    bf16x8 kf[NK], vf[NK];
    f32x4 dk[NB], dv[NB];
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
      if (kj < T) {
        a = *(const u32x4*)(kp + (size_t)kj * kvrs + 32 * ks + 8 * grp);
        c = *(const u32x4*)(vp + (size_t)kj * kvrs + 32 * ks + 8 * grp);
      }
      kf[ks] = __builtin_bit_cast(bf16x8, a);
      vf[ks] = __builtin_bit_cast(bf16x8, c);
    }
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      dk[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
      dv[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    // Steps run over (query head of the group, 64-query tile), tiles
    // fastest. The copies and the compute each keep a running cursor over
    // them (both advance one step per call, in order).
    const int i0_first = it_begin * BM, i0_last = (it_begin + n_it - 1) * BM;
    int cp_h = g * G, cp_i0 = i0_first;  // next step to copy
    int cm_i0 = i0_first;                // next step to compute
    auto issue_step = [&](int buf) {
      const int h = cp_h, i0 = cp_i0;
      if (cp_i0 == i0_last) {
        cp_i0 = i0_first;
        ++cp_h;
      } else {
        cp_i0 += BM;
      }
      const unsigned short* qp = (const unsigned short*)p.q + (size_t)b * T * qrs + (size_t)h * D;
      const unsigned short* dop = (const unsigned short*)p.dout + (size_t)b * T * qrs + (size_t)h * D;
      const BufDesc qrsr = buf_desc(qp, qspan), orsr = buf_desc(dop, qspan);
      if (i0 + BM <= T) {
        const unsigned so = (unsigned)i0 * qrs * 2u;
#pragma unroll
        for (int n = 0; n < QIPW; ++n) {
          dma16(qrsr, ld_off[n], so, lds_u32(&q_lds[buf][(wave * QIPW + n) * RPI * D]));
          dma16(orsr, ld_off[n], so, lds_u32(&do_lds[buf][(wave * QIPW + n) * RPI * D]));
        }
      } else {
#pragma unroll
        for (int n = 0; n < QIPW; ++n) {
          const int i = min(i0 + ld_row[n], T - 1);
          const unsigned vo = (unsigned)(i * qrs + ld_ch[n] * 8) * 2u;
          dma16(qrsr, vo, 0u, lds_u32(&q_lds[buf][(wave * QIPW + n) * RPI * D]));
          dma16(orsr, vo, 0u, lds_u32(&do_lds[buf][(wave * QIPW + n) * RPI * D]));
        }
      }
      if (wave < 2) {  // per-row statistics: wave 0 lse2, wave 1 delta (rows past T clamped)
        const float* src = (wave == 0 ? p.lse2 : p.delta) + ((size_t)b * p.H + h) * T;
        const int i = min(i0 + lane, T - 1);
        dma4(buf_desc(src, (unsigned)T * 4u), (unsigned)i * 4u, 0u, lds_u32(wave == 0 ? lse2_lds[buf] : dl_lds[buf]));
      }
    };

    // Copies run NBUF - 1 steps ahead; vector memory operations complete in
    // issue order, so the wait at the top of a step leaves exactly the later
    // steps' copies in flight.
    const int dma_ops = 2 * QIPW + (wave < 2 ? 1 : 0);
    auto step_fn = [&](int step, auto bufc) __attribute__((always_inline)) {
      constexpr int buf = decltype(bufc)::value;
      const int i0 = cm_i0;
      cm_i0 = cm_i0 == i0_last ? i0_first : cm_i0 + BM;
      wait_vmem_upto(dma_ops * (min(n_steps - 1, step + NBUF - 2) - step));
      lds_barrier();  // this step's tiles landed everywhere; the oldest buffer is free
      if (step + NBUF - 1 < n_steps) issue_step((buf + NBUF - 1) % NBUF);
      if (p.k_raw && step == n_steps - 1) {  // raw k row for the prologue backward
#pragma unroll
        for (int db = 0; db < NB; ++db)
          xk[db] = kj < T ? *(const u32x2*)((const unsigned short*)p.k_raw + krow + 16 * db + 4 * grp)
                          : (u32x2){0u, 0u};
      }
      const bool any = (kw <= i0 + BM - 1) && (full || kw + 15 > i0 - win);
      if (!any) return;
      const bool interior = (kw + 15 <= i0) && (full || kw > i0 + BM - 1 - win) && (i0 + BM <= T);
      const unsigned short* ql = q_lds[buf];
      const unsigned short* ol = do_lds[buf];
#pragma unroll
      for (int ib = 0; ib < BM / 32; ++ib) {
        const int rb = 32 * ib * D;
        // S and dP for queries 32 ib .. 32 ib + 31 (two 16-query blocks)
        f32x4 sacc[2], dpacc[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sacc[qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
          dpacc[qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < NK; ++ks)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const bf16x8 aq = *(const bf16x8*)(ql + aoff[ks] + rb + 16 * qb * D);
            const bf16x8 ad = *(const bf16x8*)(ol + aoff[ks] + rb + 16 * qb * D);
            sacc[qb] = mfma16(aq, kf[ks], sacc[qb]);
            dpacc[qb] = mfma16(ad, vf[ks], dpacc[qb]);
          }
        // sacc[qb][r] = S[query i0 + 32 ib + 16 qb + 4 g + r][key kj]
        f32x4 l4[2], d4[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          l4[qb] = *(const f32x4*)(&lse2_lds[buf][32 * ib + 16 * qb + 4 * grp]);
          d4[qb] = *(const f32x4*)(&dl_lds[buf][32 * ib + 16 * qb + 4 * grp]);
        }
        unsigned pw[4], sw[4];  // P and dS as bf16 pairs: B operands over the 32 queries
        auto probs = [&](auto maskc) __attribute__((always_inline)) {
          constexpr bool MASK = decltype(maskc)::value;
          const int mbase = i0 + 32 * ib + 4 * grp - kj;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            float pr[4], dsr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float pv = exp2_fast(fmaf(sacc[qb][e], p.scale_log2, -l4[qb][e]));
              if (MASK) {
                const bool vis =
                    ((unsigned)(mbase + 16 * qb + e) < wlim) && (i0 + 32 * ib + 16 * qb + 4 * grp + e < T);
                pv = vis ? pv : 0.f;
              }
              pr[e] = pv;
              dsr[e] = pv * (dpacc[qb][e] - d4[qb][e]);
            }
            pw[2 * qb] = pk_bf16(pr[0], pr[1]);
            pw[2 * qb + 1] = pk_bf16(pr[2], pr[3]);
            sw[2 * qb] = pk_bf16(dsr[0], dsr[1]);
            sw[2 * qb + 1] = pk_bf16(dsr[2], dsr[3]);
          }
        };
        if (interior)
          probs(std::integral_constant<bool, false>{});
        else
          probs(std::integral_constant<bool, true>{});
        const bf16x8 pb = __builtin_bit_cast(bf16x8, (u32x4){pw[0], pw[1], pw[2], pw[3]});
        const bf16x8 sb = __builtin_bit_cast(bf16x8, (u32x4){sw[0], sw[1], sw[2], sw[3]});
        // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          const bf16x8 ot = cat_bf16x8(lds_read_tr16(ol + toff[db] + rb), lds_read_tr16(ol + toff[db] + rb + 16 * D));
          const bf16x8 qt = cat_bf16x8(lds_read_tr16(ql + toff[db] + rb), lds_read_tr16(ql + toff[db] + rb + 16 * D));
          dv[db] = mfma16(ot, pb, dv[db]);
          dk[db] = mfma16(qt, sb, dk[db]);
        }
      }
    };
#pragma unroll
    for (int s = 0; s < NBUF - 1; ++s)
      if (s < n_steps) issue_step(s);
    for (int step = 0; step < n_steps; step += NBUF) {
      step_fn(step, std::integral_constant<int, 0>{});
      if constexpr (NBUF > 1)
        if (step + 1 < n_steps) step_fn(step + 1, std::integral_constant<int, 1 % NBUF>{});
      if constexpr (NBUF > 2)
        if (step + 2 < n_steps) step_fn(step + 2, std::integral_constant<int, 2 % NBUF>{});
    }

    store_grad_row16<D>(p, dv, 1.0f, kj < T, nullptr, 0, grp, (unsigned short*)p.dv + krow);
    store_grad_row16<D>(p, dk, p.scale, kj < T, p.k_raw ? xk : nullptr, kj + (p.pos_offset ? p.pos_offset[b] : 0),
                        grp, (unsigned short*)p.dk + krow);
  };

  // one copy of the tile code for both key tiles of a pair
  const int n_pass = PAIRED && nkt - 1 - r_pair > r_pair ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    if (pass) lds_barrier();  // every wave is done with the last step's tiles before they are reloaded
    run(pass ? nkt - 1 - r_pair : r_pair);
  }
}

// --------------------------------------------------------------------------
// dQ: one workgroup per (b, h, 128-query tile), 4 waves of 32 queries; K/V
// tiles of 64 keys stream through double-buffered LDS as in the forward.
template <int D>
__global__ __launch_bounds__(BWD_THREADS, 2) void attn_bwd_dq_kernel(BwdParams p) {
  constexpr int NC = D / 8;
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int TILE = DQ_BN * D;       // elements of one K or V tile
  constexpr int RPI = 64 / NC;          // tile rows per direct-to-LDS instruction
  constexpr int IPW = DQ_BN / RPI / 4;  // such instructions per wave per tensor per tile
  static_assert(IPW >= 1 && DQ_BN % (4 * RPI) == 0, "tile/wave mismatch");
  __shared__ __attribute__((aligned(16))) unsigned short kv_lds[2][2][TILE];

  const int T = p.T;
  const int nqt = (T + DQ_BM - 1) / DQ_BM;
  const int N = nqt * p.H * p.B;
  const int logical = xcd_remap(blockIdx.x, N);
  const int bh = logical / nqt;
  const int qt = nqt - 1 - (logical - bh * nqt);  // late (heavier) query tiles first
  const int b = bh / p.H, h = bh - b * p.H;
  const int g = h / (p.H / p.Hkv);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, hh = lane >> 5;
  const int grp = lane >> 4, t16 = lane & 15;
  const int q0 = qt * DQ_BM;
  const int qw = q0 + wave * 32;
  const int qi = qw + li;
  const bool q_valid = qi < T;

  const size_t qrs = (size_t)p.H * D;
  const unsigned kvrs = (unsigned)(p.Hkv * D);
  const unsigned short* qp = (const unsigned short*)p.q + (size_t)b * T * qrs + (size_t)h * D;
  const unsigned short* dop = (const unsigned short*)p.dout + (size_t)b * T * qrs + (size_t)h * D;
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)b * T * kvrs + (size_t)g * D;
  const unsigned short* vp = (const unsigned short*)p.v + (size_t)b * T * kvrs + (size_t)g * D;
  const unsigned span = (unsigned)(((size_t)(T - 1) * kvrs + D) * 2);
  const BufDesc krs = buf_desc(kp, span), vrs = buf_desc(vp, span);

  // q and dO as B operands of S^T = K Q^T and dP^T = V dO^T: lane (li, hh)
  // holds x[qi][16 s + 8 hh + e]; the lane's row statistics.
  bf16x8 qf[NS], of[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (q_valid) {
      a = *(const u32x4*)(qp + (size_t)qi * qrs + 16 * s + 8 * hh);
      c = *(const u32x4*)(dop + (size_t)qi * qrs + 16 * s + 8 * hh);
    }
    qf[s] = __builtin_bit_cast(bf16x8, a);
    of[s] = __builtin_bit_cast(bf16x8, c);
  }
  // This lane's row statistics, formed here and also stored for the dK/dV
  // kernel that runs next: delta = <dout, out> (the two half-waves hold the
  // two halves of d) and lse * log2(e).
  const size_t si = ((size_t)b * p.H + h) * T + (q_valid ? qi : 0);
  float dl = 0.f;
  if (q_valid) {
    const unsigned short* opr = (const unsigned short*)p.out + ((size_t)b * T + qi) * qrs + (size_t)h * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float o8[8], d8[8];
      unpack8_bf16(*(const u32x4*)(opr + 16 * s + 8 * hh), o8);
      unpack8_bf16(__builtin_bit_cast(u32x4, of[s]), d8);
#pragma unroll
      for (int e = 0; e < 8; ++e) dl = fmaf(d8[e], o8[e], dl);
    }
  }
  dl = sum_mod<32>(dl);
  const float l2 = q_valid ? p.lse[si] * kLog2e : 0.f;
  if (q_valid && hh == 0) {
    p.delta[si] = dl;
    p.lse2[si] = l2;
  }

  const bool full = p.window <= 0;
  const int win = p.window;
  const unsigned wlim = full ? 0x80000000u : (unsigned)win;  // key j visible to i iff (unsigned)(i - j) < wlim
  const int kv_hi = min(T - 1, q0 + DQ_BM - 1);
  const int kv_lo = full ? 0 : max(0, q0 - win + 1);
  const int t_begin = kv_lo / DQ_BN, t_end = kv_hi / DQ_BN;

  unsigned ld_off[IPW];
  int ld_row[IPW], ld_ch[IPW];
#pragma unroll
  for (int n = 0; n < IPW; ++n) {
    const int row = (wave * IPW + n) * RPI + lane / NC;
    ld_row[n] = row;
    ld_ch[n] = (lane % NC) ^ (swz<NC>(row) & (NC - 1));
    ld_off[n] = (unsigned)(row * kvrs + ld_ch[n] * 8) * 2u;
  }
  auto issue_tile = [&](int jt, int buf) {
    const int j0 = jt * DQ_BN;
    if (j0 + DQ_BN <= T) {
      const unsigned so = (unsigned)j0 * kvrs * 2u;
#pragma unroll
      for (int n = 0; n < IPW; ++n) {
        dma16(krs, ld_off[n], so, lds_u32(&kv_lds[buf][0][(wave * IPW + n) * RPI * D]));
        dma16(vrs, ld_off[n], so, lds_u32(&kv_lds[buf][1][(wave * IPW + n) * RPI * D]));
      }
    } else {  // last tile: rows past T clamped to T - 1 (masked by causality)
#pragma unroll
      for (int n = 0; n < IPW; ++n) {
        const int j = min(j0 + ld_row[n], T - 1);
        const unsigned vo = (unsigned)(j * kvrs + ld_ch[n] * 8) * 2u;
        dma16(krs, vo, 0u, lds_u32(&kv_lds[buf][0][(wave * IPW + n) * RPI * D]));
        dma16(vrs, vo, 0u, lds_u32(&kv_lds[buf][1][(wave * IPW + n) * RPI * D]));
      }
    }
  };

  // K and V rows li (+32 jb) at chunk 2 st + hh (A operands); K^T transpose
  // reads at rows 4 hh + t16/4 (+8) (+16 u + 32 jb), columns 32 d + 16 (grp & 1) + 4 (t16 & 3).
  int koff[NS], toff1[ND], toff2[ND];
#pragma unroll
  for (int st = 0; st < NS; ++st) koff[st] = swz_off<NC>(li, 16 * st + 8 * hh);
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const int col = 32 * d + 16 * (grp & 1) + 4 * (t16 & 3);
    toff1[d] = swz_off<NC>(4 * hh + (t16 >> 2), col);
    toff2[d] = swz_off<NC>(4 * hh + (t16 >> 2) + 8, col);
  }

  f32x16 acc[ND];  // dQ^T: acc[d][r] = dq[qi][32 d + 8 (r/4) + 4 hh + r%4] / scale
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = (f32x16){};

  auto tile = [&](int jt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmem();    // this wave's copies of tile jt (the only loads in flight)
    lds_barrier();  // everyone's copies of tile jt landed; the other buffer is free
    if (jt < t_end) issue_tile(jt + 1, buf ^ 1);
    const unsigned short* kl = kv_lds[buf][0];
    const unsigned short* vl = kv_lds[buf][1];

    const int j0 = jt * DQ_BN;
    const bool any = (j0 <= qw + 31) && (full || j0 + DQ_BN - 1 > qw - win);
    if (!any) return;
    const bool interior = (j0 + DQ_BN - 1 <= qw) && (full || j0 > qw + 31 - win);

    f32x16 s[2] = {(f32x16){}, (f32x16){}}, dp[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const bf16x8 a = *(const bf16x8*)(kl + koff[st] + jb * 32 * D);
        const bf16x8 c = *(const bf16x8*)(vl + koff[st] + jb * 32 * D);
        s[jb] = mfma32(a, qf[st], s[jb]);
        dp[jb] = mfma32(c, of[st], dp[jb]);
      }
    // s[jb][r] = S[key j0 + 32 jb + 8 (r/4) + 4 hh + r%4][query qi]; dS^T as bf16 pairs
    unsigned dw[2][8];
    auto grads = [&](auto maskc) {
      constexpr bool MASK = decltype(maskc)::value;
      const int base = qi - j0 - 4 * hh;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float ds[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float pv = exp2_fast(fmaf(s[jb][r + e], p.scale_log2, -l2));
            if (MASK && (unsigned)(base - (32 * jb + 8 * ((r + e) >> 2) + ((r + e) & 3))) >= wlim) pv = 0.f;
            ds[e] = pv * (dp[jb][r + e] - dl);
          }
          dw[jb][r >> 1] = pk_bf16(ds[0], ds[1]);
        }
    };
    if (interior)
      grads(std::integral_constant<bool, false>{});
    else
      grads(std::integral_constant<bool, true>{});

    // dQ^T += K^T dS^T over the tile's 64 keys.
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 sq = {dw[jb][4 * u], dw[jb][4 * u + 1], dw[jb][4 * u + 2], dw[jb][4 * u + 3]};
        const bf16x8 sb = __builtin_bit_cast(bf16x8, sq);
        const int rb = (32 * jb + 16 * u) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const s16x4 x1 = lds_read_tr16(kl + toff1[d] + rb);
          const s16x4 x2 = lds_read_tr16(kl + toff2[d] + rb);
          acc[d] = mfma32(cat_bf16x8(x1, x2), sb, acc[d]);
        }
      }
  };

  issue_tile(t_begin, 0);
  for (int jt = t_begin; jt <= t_end; jt += 2) {
    tile(jt, std::integral_constant<int, 0>{});
    if (jt + 1 <= t_end) tile(jt + 1, std::integral_constant<int, 1>{});
  }

  // dq (through the prologue backward when asked) for this lane's query (its
  // raw q row is loaded here: requesting it earlier costs registers the tile
  // loop needs)
  const size_t qrow = ((size_t)b * T + qi) * qrs + (size_t)h * D;
  u32x2 xq[ND * 4];
  if (p.q_raw) load_row_words<D>((const unsigned short*)p.q_raw + qrow, q_valid, hh, xq);
  store_grad_row<D>(p, acc, p.scale, q_valid, p.q_raw ? xq : nullptr, qi + (p.pos_offset ? p.pos_offset[b] : 0),
                    hh, (unsigned short*)p.dq + qrow);
}

// --------------------------------------------------------------------------
// float32 backward: (dk, dv) per key, then dq per query, plain loops.
template <int D>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(BwdParams p) {
  const int T = p.T;
  const int j = blockIdx.x * 64 + threadIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  if (j >= T) return;
  const int G = p.H / p.Hkv;
  const size_t kvrs = (size_t)p.Hkv * D, qrs = (size_t)p.H * D;
  const float* kr = (const float*)p.k + ((size_t)b * T + j) * kvrs + (size_t)g * D;
  const float* vr = (const float*)p.v + ((size_t)b * T + j) * kvrs + (size_t)g * D;
  float kk[D], vv[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kk[d] = kr[d];
    vv[d] = vr[d];
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const int hi = p.window <= 0 ? T - 1 : min(T - 1, j + p.window - 1);
  for (int hq = 0; hq < G; ++hq) {
    const int h = g * G + hq;
    for (int i = j; i <= hi; ++i) {
      const float* qi = (const float*)p.q + ((size_t)b * T + i) * qrs + (size_t)h * D;
      const float* doi = (const float*)p.dout + ((size_t)b * T + i) * qrs + (size_t)h * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(qi[d], kk[d], s);
        dp = fmaf(doi[d], vv[d], dp);
      }
      const size_t li = ((size_t)b * p.H + h) * T + i;
      const float pr = expf(s * p.scale - p.lse[li]);
      const float ds = pr * (dp - p.delta[li]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dv[d] = fmaf(pr, doi[d], dv[d]);
        dk[d] = fmaf(ds, qi[d], dk[d]);
      }
    }
  }
  float* dkp = (float*)p.dk + ((size_t)b * T + j) * kvrs + (size_t)g * D;
  float* dvp = (float*)p.dv + ((size_t)b * T + j) * kvrs + (size_t)g * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    dkp[d] = dk[d] * p.scale;
    dvp[d] = dv[d];
  }
}

template <int D>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(BwdParams p) {
  const int T = p.T;
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= T) return;
  const int g = h / (p.H / p.Hkv);
  const size_t kvrs = (size_t)p.Hkv * D, qrs = (size_t)p.H * D;
  const float* qi = (const float*)p.q + ((size_t)b * T + i) * qrs + (size_t)h * D;
  const float* doi = (const float*)p.dout + ((size_t)b * T + i) * qrs + (size_t)h * D;
  float qq[D], dd[D], dq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qq[d] = qi[d];
    dd[d] = doi[d];
    dq[d] = 0.f;
  }
  const size_t li = ((size_t)b * p.H + h) * T + i;
  const float lse = p.lse[li], delta = p.delta[li];
  const int lo = p.window <= 0 ? 0 : max(0, i - p.window + 1);
  for (int j = lo; j <= i; ++j) {
    const float* kr = (const float*)p.k + ((size_t)b * T + j) * kvrs + (size_t)g * D;
    const float* vr = (const float*)p.v + ((size_t)b * T + j) * kvrs + (size_t)g * D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      s = fmaf(qq[d], kr[d], s);
      dp = fmaf(dd[d], vr[d], dp);
    }
    const float pr = expf(s * p.scale - lse);
    const float ds = pr * (dp - delta);
#pragma unroll
    for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, kr[d], dq[d]);
  }
  float* dqp = (float*)p.dq + ((size_t)b * T + i) * qrs + (size_t)h * D;
#pragma unroll
  for (int d = 0; d < D; ++d) dqp[d] = dq[d] * p.scale;
}


template <int D>
hipError_t launch_pre(const BwdParams& p, hipStream_t s) {
  const long threads = (long)p.B * p.T * p.H * (D / 8);
  bwd_pre_f32_kernel<D><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t record(hipEvent_t ev, hipStream_t s) { return ev ? hipEventRecord(ev, s) : hipSuccess; }

template <int D>
hipError_t launch_bf16(const BwdParams& p, hipStream_t s, const BwdEvents& ev) {
  hipError_t e;
  // the dQ kernel first: it also forms the row statistics the dK/dV kernel reads
  if ((e = record(ev.dq_begin, s)) != hipSuccess) return e;
  const int nqt = (p.T + DQ_BM - 1) / DQ_BM;
  attn_bwd_dq_kernel<D><<<nqt * p.H * p.B, BWD_THREADS, 0, s>>>(p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = record(ev.dkdv_begin, s)) != hipSuccess) return e;
  const int nkt = (p.T + K16_BN - 1) / K16_BN;
  if (p.window <= 0)
    attn_bwd_dkdv16_kernel<D, true><<<(nkt + 1) / 2 * p.Hkv * p.B, BWD16_THREADS, 0, s>>>(p);
  else
    attn_bwd_dkdv16_kernel<D, false><<<nkt * p.Hkv * p.B, BWD16_THREADS, 0, s>>>(p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record(ev.end, s);
}

template <int D>
hipError_t launch_f32(const BwdParams& p, hipStream_t s, const BwdEvents& ev) {
  hipError_t e = launch_pre<D>(p, s);
  if (e != hipSuccess) return e;
  if ((e = record(ev.dq_begin, s)) != hipSuccess) return e;
  bwd_dq_f32_kernel<D><<<dim3((p.T + 63) / 64, p.H, p.B), 64, 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = record(ev.dkdv_begin, s)) != hipSuccess) return e;
  bwd_dkdv_f32_kernel<D><<<dim3((p.T + 63) / 64, p.Hkv, p.B), 64, 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return record(ev.end, s);
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdParams& p, hipStream_t s, const BwdEvents& ev) {
  switch (p.D) {
    case 32: return launch_bf16<32>(p, s, ev);
    case 64: return launch_bf16<64>(p, s, ev);
    case 128: return launch_bf16<128>(p, s, ev);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_f32(const BwdParams& p, hipStream_t s, const BwdEvents& ev) {
  switch (p.D) {
    case 32: return launch_f32<32>(p, s, ev);
    case 64: return launch_f32<64>(p, s, ev);
    case 128: return launch_f32<128>(p, s, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
