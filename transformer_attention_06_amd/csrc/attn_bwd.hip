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
// bf16 path, three kernels:
//   pre:  delta_i = <dout_i, out_i> and lse_i * log2(e) in float32; clear the
//         float32 dq accumulator.
//   main: one workgroup per (b, kv head, 128-key tile); each of the 4 waves
//         keeps 32 keys' K and V fragments in registers and accumulates dK^T
//         and dV^T for them over every query head of the GQA group and every
//         64-query tile that intersects the band. S = Q K^T and dP = dO V^T
//         come out with one key column per lane, which is directly the
//         B-operand layout of dV^T += dO^T P and dK^T += Q^T dS; dO^T and
//         Q^T are LDS transpose reads. dS goes through LDS once so that
//         dQ = dS K for the 128 keys is formed per workgroup (each wave owns
//         one 32-wide slice of d, whose K^T operand stays in registers) and
//         added to the float32 accumulator with buffer atomics. Q/dO tiles
//         and the per-row statistics stream into double-buffered LDS with
//         buffer-to-LDS loads; LDS addresses are per-lane constants.
//   post: dq = bf16(scale-applied accumulator).
// f32 path: plain per-key (dk, dv) and per-query (dq) loops in float32.

#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace nc {
namespace {

constexpr int BWD_BN = 128;  // keys per workgroup (32 per wave)
constexpr int BWD_BM = 64;   // queries per step
constexpr int BWD_THREADS = 256;
constexpr int NBUF = 3;  // q/dO tile buffers: loads run two steps ahead

// --------------------------------------------------------------------------
// delta = rowsum(dout * out), lse2 = lse * log2(e) (float32), dq_acc := 0.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const long rows = (long)p.B * p.T * p.H;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long row = gid / LPR;
  const int c = (int)(gid - row * LPR);
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + c * 8;
    float a[8], o[8];
    if (BF16) {
      unpack8_bf16(*(const u32x4*)((const unsigned short*)p.dout + off), a);
      unpack8_bf16(*(const u32x4*)((const unsigned short*)p.out + off), o);
    } else {
      const f32x4* pa = (const f32x4*)((const float*)p.dout + off);
      const f32x4* po = (const f32x4*)((const float*)p.out + off);
      const f32x4 a0 = pa[0], a1 = pa[1], o0 = po[0], o1 = po[1];
      for (int i = 0; i < 4; ++i) {
        a[i] = a0[i];
        a[4 + i] = a1[i];
        o[i] = o0[i];
        o[4 + i] = o1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(a[i], o[i], acc);
    if (p.dq_acc) {
      f32x4* z = (f32x4*)(p.dq_acc + off);
      z[0] = (f32x4){};
      z[1] = (f32x4){};
    }
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

// dq = bf16(dq_acc) (the accumulator already carries the scale).
__global__ __launch_bounds__(256) void bwd_post_kernel(const float* __restrict__ acc,
                                                       unsigned short* __restrict__ dq, long n8) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4* a = (const f32x4*)(acc + i * 8);
  const f32x4 a0 = a[0], a1 = a[1];
  const float f[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  *(u32x4*)(dq + i * 8) = pack8_bf16(f);
}

// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(BWD_THREADS, 1) void attn_bwd_bf16_kernel(BwdParams p) {
  constexpr int NC = D / 8;        // chunks per row of the q/dO/K tiles (swizzled)
  constexpr int NCS = BWD_BM / 8;  // chunks per row of the dS^T tile [key][query]
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int QT = BWD_BM * D;   // elements of one q or dO tile
  constexpr int RPI = 64 / NC;     // tile rows per direct-to-LDS instruction
  constexpr int QIPW = BWD_BM / RPI / 4;   // such instructions per wave per tensor
  constexpr int KIPW = BWD_BN / RPI / 4;
  static_assert(QIPW >= 1 && KIPW >= 1, "tile/wave mismatch");
  static_assert(2 * QT >= BWD_BN * D, "K staging must fit in the q tile buffers");
  // q/dO tiles double-buffered; the K tile is staged once in q_lds at start
  __shared__ __attribute__((aligned(16))) unsigned short q_lds[NBUF][QT];
  __shared__ __attribute__((aligned(16))) unsigned short do_lds[NBUF][QT];
  __shared__ __attribute__((aligned(16))) unsigned short ds_lds[BWD_BN * BWD_BM];
  __shared__ __attribute__((aligned(16))) float lse2_lds[NBUF][BWD_BM];
  __shared__ __attribute__((aligned(16))) float dl_lds[NBUF][BWD_BM];

  const int T = p.T;
  const int nkt = (T + BWD_BN - 1) / BWD_BN;
  const int N = nkt * p.Hkv * p.B;
  const int logical = xcd_remap(blockIdx.x, N);
  const int bg = logical / nkt;
  const int kt = logical - bg * nkt;  // early key tiles (most queries) first
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int G = p.H / p.Hkv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, hh = lane >> 5;
  const int grp = lane >> 4, t16 = lane & 15;
  const int j0 = kt * BWD_BN;
  const int kw = j0 + wave * 32;
  const int kj = kw + li;  // this lane's key

  const unsigned qrs = (unsigned)(p.H * D);
  const unsigned kvrs = (unsigned)(p.Hkv * D);
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)b * T * kvrs + (size_t)g * D;
  const unsigned short* vp = (const unsigned short*)p.v + (size_t)b * T * kvrs + (size_t)g * D;

  // ---- K tile -> LDS (rows past T clamped), then K^T fragments for dQ ----
  // This wave forms dQ for d in [32 dbw, 32 dbw + 32); ktf[u] holds the B
  // operand K[16 u + 8 hh + e][32 dbw + li] for the 16-key step u.
  const int dbw = wave % ND;
  {
    const BufDesc krs = buf_desc(kp, (unsigned)(((size_t)(T - 1) * kvrs + D) * 2));
#pragma unroll
    for (int n = 0; n < KIPW; ++n) {
      const int inst = wave * KIPW + n;
      const int row = inst * RPI + lane / NC;
      const int ch = (lane % NC) ^ (swz<NC>(row) & (NC - 1));
      const int j = min(j0 + row, T - 1);
      dma16(krs, (unsigned)(j * kvrs + ch * 8) * 2u, 0u, lds_u32(&q_lds[0][inst * RPI * D]));
    }
  }
  // K and V fragments of this lane's key: lane (li, hh) holds x[kj][16 s + 8 hh + e].
  bf16x8 kf[NS], vf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (kj < T) {
      a = *(const u32x4*)(kp + (size_t)kj * kvrs + 16 * s + 8 * hh);
      c = *(const u32x4*)(vp + (size_t)kj * kvrs + 16 * s + 8 * hh);
    }
    kf[s] = __builtin_bit_cast(bf16x8, a);
    vf[s] = __builtin_bit_cast(bf16x8, c);
  }
  const int tr_row = t16 >> 2;
  const int tr_col = 16 * (grp & 1) + 4 * (t16 & 3);
  wait_vmem();
  lds_barrier();
  bf16x8 ktf[BWD_BN / 16];
  {
    const unsigned short* kl = q_lds[0];
#pragma unroll
    for (int u = 0; u < BWD_BN / 16; ++u) {
      const int r0 = 16 * u + 8 * hh + tr_row;
      const s16x4 b1 = lds_read_tr16(kl + swz_off<NC>(r0, 32 * dbw + tr_col));
      const s16x4 b2 = lds_read_tr16(kl + swz_off<NC>(r0 + 4, 32 * dbw + tr_col));
      ktf[u] = cat_bf16x8(b1, b2);
    }
  }
  lds_barrier();  // every wave has its K^T fragments before q/dO tiles overwrite the staging area

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    dk[d] = (f32x16){};
    dv[d] = (f32x16){};
  }

  const bool full = p.window <= 0;
  const int win = p.window;
  const unsigned wlim = full ? 0x80000000u : (unsigned)win;
  const int i_last = full ? T - 1 : min(T - 1, j0 + BWD_BN - 1 + win - 1);
  const int it_begin = j0 / BWD_BM, n_it = i_last / BWD_BM - it_begin + 1;
  const int n_steps = G * n_it;

  // ---- per-lane constant LDS offsets ----
  // q/dO operand rows li (+32 ib) at chunk 2 st + hh
  int aoff[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) aoff[st] = swz_off<NC>(li, 16 * st + 8 * hh);
  // transpose reads of dO^T / Q^T: rows 4 hh + t16/4 (+8) (+16 u + 32 ib), columns 32 d + tr_col
  int toff1[ND], toff2[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    toff1[d] = swz_off<NC>(4 * hh + tr_row, 32 * d + tr_col);
    toff2[d] = swz_off<NC>(4 * hh + tr_row + 8, 32 * d + tr_col);
  }
  // dS^T transpose reads for dQ: rows 16 u + 8 hh + t16/4 (+4), columns 32 ib + tr_col
  int soff1[2], soff2[2];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib) {
    soff1[ib] = swz_off<NCS>(8 * hh + tr_row, 32 * ib + tr_col);
    soff2[ib] = swz_off<NCS>(8 * hh + tr_row + 4, 32 * ib + tr_col);
  }
  // dS^T stores: row wave*32 + li, columns 32 ib + 8 rg + 4 hh
  int woff[2][4];
#pragma unroll
  for (int ib = 0; ib < 2; ++ib)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) woff[ib][rg] = swz_off<NCS>(wave * 32 + li, 32 * ib + 8 * rg + 4 * hh);

  // ---- q/dO tile loads (buffer -> LDS) ----
  unsigned ld_off[QIPW];
  int ld_row[QIPW], ld_ch[QIPW];
#pragma unroll
  for (int n = 0; n < QIPW; ++n) {
    const int row = (wave * QIPW + n) * RPI + lane / NC;
    ld_row[n] = row;
    ld_ch[n] = (lane % NC) ^ (swz<NC>(row) & (NC - 1));
    ld_off[n] = (unsigned)(row * qrs + ld_ch[n] * 8) * 2u;
  }
  const unsigned qspan = (unsigned)(((size_t)(T - 1) * qrs + D) * 2);
  auto issue_step = [&](int step, int buf) {
    const int hq = step / n_it;
    const int i0 = (it_begin + step - hq * n_it) * BWD_BM;
    const int h = g * G + hq;
    const unsigned short* qp = (const unsigned short*)p.q + (size_t)b * T * qrs + (size_t)h * D;
    const unsigned short* dop = (const unsigned short*)p.dout + (size_t)b * T * qrs + (size_t)h * D;
    const BufDesc qrsr = buf_desc(qp, qspan), orsr = buf_desc(dop, qspan);
    if (i0 + BWD_BM <= T) {
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

  // dQ accumulator rows (buffer atomics): voffset per (ib), soffset per (step, r)
  const int n_qb = (2 * ND + 3 - wave) / 4;  // dQ blocks of this wave: n = wave + 4 m < 2 ND
  const int ib_first = wave / ND;            // ib of block m is ib_first + m (ND = 4: 0, 1)

  // The dQ atomics of a step stay in flight into the next step: the wait at
  // the top of a step only covers the loads issued before those atomics
  // (vector memory operations complete in issue order).
  // Vector memory operations complete in issue order, so the wait at the top
  // of step t only has to cover the tile loads of step t: the loads of step
  // t+1 and the dQ atomics of steps t-2 and t-1, issued after them, may stay
  // in flight.
  const int dma_ops = 2 * QIPW + (wave < 2 ? 1 : 0);  // loads this wave issues per step
  int at_prev2 = 0, at_prev1 = 0;                     // atomics of steps t-2, t-1
  int pending = 0;                                    // atomics of the current step (0 if unknown)
  issue_step(0, 0);
  if (n_steps > 1) issue_step(1, 1);
  auto step_fn = [&](int step, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int hq = step / n_it;
    const int i0 = (it_begin + step - hq * n_it) * BWD_BM;
    const int h = g * G + hq;
    wait_vmem_upto(at_prev2 + at_prev1 + (step + 1 < n_steps ? dma_ops : 0));
    lds_barrier();  // step's tiles landed; previous dQ readers are done with ds_lds
    if (step + 2 < n_steps) issue_step(step + 2, (buf + 2) % NBUF);
    const unsigned short* ql = q_lds[buf];
    const unsigned short* ol = do_lds[buf];

    const bool any = (kw <= i0 + BWD_BM - 1) && (full || kw + 31 > i0 - win);
    const bool interior = (kw + 31 <= i0) && (full || kw > i0 + BWD_BM - 1 - win) && (i0 + BWD_BM <= T);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      unsigned sw[8];  // dS as bf16 pairs
      if (any) {
        // Every LDS operand of this 32-query half is requested before the
        // first product: q and dO rows (S, dP), the row statistics, and the
        // dO^T / Q^T transpose reads (dV, dK).
        bf16x8 aq[NS], ad[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          aq[st] = *(const bf16x8*)(ql + aoff[st] + 32 * ib * D);
          ad[st] = *(const bf16x8*)(ol + aoff[st] + 32 * ib * D);
        }
        f32x4 l4[4], d4[4];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          l4[rg] = *(const f32x4*)(&lse2_lds[buf][32 * ib + 8 * rg + 4 * hh]);
          d4[rg] = *(const f32x4*)(&dl_lds[buf][32 * ib + 8 * rg + 4 * hh]);
        }
        bf16x8 ot[2][ND], qt[2][ND];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const int rb = (32 * ib + 16 * u) * D;
            ot[u][d] = cat_bf16x8(lds_read_tr16(ol + toff1[d] + rb), lds_read_tr16(ol + toff2[d] + rb));
            qt[u][d] = cat_bf16x8(lds_read_tr16(ql + toff1[d] + rb), lds_read_tr16(ql + toff2[d] + rb));
          }

        f32x16 sacc = (f32x16){}, dpacc = (f32x16){};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          sacc = mfma32(aq[st], kf[st], sacc);
          dpacc = mfma32(ad[st], vf[st], dpacc);
        }
        // sacc[r] = S[query i0 + 32 ib + 8 (r/4) + 4 hh + r%4][key kj]
        unsigned pw[8];
        auto probs = [&](auto maskc) {
          constexpr bool MASK = decltype(maskc)::value;
          const int mbase = i0 + 32 * ib + 4 * hh - kj;
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            float pr[4], dsr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * rg + e;
              float pv = exp2_fast(fmaf(sacc[r], p.scale_log2, -l4[rg][e]));
              if (MASK) {
                const int off = 8 * rg + e;
                const bool vis = ((unsigned)(mbase + off) < wlim) && (i0 + 32 * ib + 8 * rg + 4 * hh + e < T);
                pv = vis ? pv : 0.f;
              }
              pr[e] = pv;
              dsr[e] = pv * (dpacc[r] - d4[rg][e]);
            }
            pw[2 * rg] = pk_bf16(pr[0], pr[1]);
            pw[2 * rg + 1] = pk_bf16(pr[2], pr[3]);
            sw[2 * rg] = pk_bf16(dsr[0], dsr[1]);
            sw[2 * rg + 1] = pk_bf16(dsr[2], dsr[3]);
          }
        };
        if (interior)
          probs(std::integral_constant<bool, false>{});
        else
          probs(std::integral_constant<bool, true>{});
        // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 pq = {pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]};
          const u32x4 sq = {sw[4 * u], sw[4 * u + 1], sw[4 * u + 2], sw[4 * u + 3]};
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pq);
          const bf16x8 sb = __builtin_bit_cast(bf16x8, sq);
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            dv[d] = mfma32(ot[u][d], pb, dv[d]);
            dk[d] = mfma32(qt[u][d], sb, dk[d]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) sw[i] = 0u;
      }
      // dS^T -> LDS: row = key (wave*32 + li), 4 consecutive queries per store.
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) *(u32x2*)(ds_lds + woff[ib][rg]) = (u32x2){sw[2 * rg], sw[2 * rg + 1]};
    }
    lds_barrier();

    // dQ[i][d] = sum over the 128 keys of dS[i][j] K[j][d] for this wave's
    // d slice; added to the float32 accumulator rows i0 .. i0+63 of head h.
    float* dqa = p.dq_acc + (size_t)b * T * qrs + (size_t)h * D;
    const __amdgpu_buffer_rsrc_t dqr = make_rsrc(dqa, (unsigned)((size_t)T * qrs * 4));
    pending = 0;
    for (int m = 0; m < n_qb; ++m) {
      const int ib = ib_first + m;
      f32x16 acc = (f32x16){};
#pragma unroll
      for (int u = 0; u < BWD_BN / 16; ++u) {
        const int rb = 16 * u * BWD_BM;
        const s16x4 a1 = lds_read_tr16(ds_lds + (ib ? soff1[1] : soff1[0]) + rb);
        const s16x4 a2 = lds_read_tr16(ds_lds + (ib ? soff2[1] : soff2[0]) + rb);
        acc = mfma32(cat_bf16x8(a1, a2), ktf[u], acc);
      }
      // acc[r] = dQ[query i0 + 32 ib + 8 (r/4) + 4 hh + r%4][d = 32 dbw + li]
      const unsigned vo = (unsigned)((32 * ib + 4 * hh) * qrs + 32 * dbw + li) * 4u;
      if (i0 + BWD_BM <= T) {
        pending += 16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const unsigned so = (unsigned)(i0 + 8 * (r >> 2) + (r & 3)) * qrs * 4u;
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r] * p.scale, dqr, vo, so, 0);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + 32 * ib + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (i < T) {
            const unsigned so = (unsigned)(i0 + 8 * (r >> 2) + (r & 3)) * qrs * 4u;
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r] * p.scale, dqr, vo, so, 0);
          }
        }
      }
    }
    at_prev2 = at_prev1;
    at_prev1 = pending;
  };

  for (int step = 0; step < n_steps; step += NBUF) {
    step_fn(step, std::integral_constant<int, 0>{});
    if (step + 1 < n_steps) step_fn(step + 1, std::integral_constant<int, 1>{});
    if (step + 2 < n_steps) step_fn(step + 2, std::integral_constant<int, 2>{});
  }

  // dK (scaled) and dV for this lane's key.
  if (kj < T) {
    unsigned short* dkp = (unsigned short*)p.dk + ((size_t)b * T + kj) * kvrs + (size_t)g * D;
    unsigned short* dvp = (unsigned short*)p.dv + ((size_t)b * T + kj) * kvrs + (size_t)g * D;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 wk, wv;
        wk[0] = pk_bf16(dk[d][4 * rg] * p.scale, dk[d][4 * rg + 1] * p.scale);
        wk[1] = pk_bf16(dk[d][4 * rg + 2] * p.scale, dk[d][4 * rg + 3] * p.scale);
        wv[0] = pk_bf16(dv[d][4 * rg], dv[d][4 * rg + 1]);
        wv[1] = pk_bf16(dv[d][4 * rg + 2], dv[d][4 * rg + 3]);
        *(u32x2*)(dkp + 32 * d + 8 * rg + 4 * hh) = wk;
        *(u32x2*)(dvp + 32 * d + 8 * rg + 4 * hh) = wv;
      }
  }
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


template <int D, bool BF16>
hipError_t launch_pre(const BwdParams& p, hipStream_t s) {
  const long threads = (long)p.B * p.T * p.H * (D / 8);
  bwd_pre_kernel<D, BF16><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t record(hipEvent_t ev, hipStream_t s) { return ev ? hipEventRecord(ev, s) : hipSuccess; }

template <int D>
hipError_t launch_bf16(const BwdParams& p, hipStream_t s, hipEvent_t eb, hipEvent_t ee) {
  hipError_t e = launch_pre<D, true>(p, s);
  if (e != hipSuccess) return e;
  const int nkt = (p.T + BWD_BN - 1) / BWD_BN;
  if ((e = record(eb, s)) != hipSuccess) return e;
  attn_bwd_bf16_kernel<D><<<nkt * p.Hkv * p.B, BWD_THREADS, 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = record(ee, s)) != hipSuccess) return e;
  const long n8 = (long)p.B * p.T * p.H * D / 8;
  bwd_post_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(p.dq_acc, (unsigned short*)p.dq, n8);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const BwdParams& p, hipStream_t s, hipEvent_t eb, hipEvent_t ee) {
  hipError_t e = launch_pre<D, false>(p, s);
  if (e != hipSuccess) return e;
  if ((e = record(eb, s)) != hipSuccess) return e;
  bwd_dkdv_f32_kernel<D><<<dim3((p.T + 63) / 64, p.Hkv, p.B), 64, 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_dq_f32_kernel<D><<<dim3((p.T + 63) / 64, p.H, p.B), 64, 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return record(ee, s);
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdParams& p, hipStream_t s, hipEvent_t eb, hipEvent_t ee) {
  switch (p.D) {
    case 32: return launch_bf16<32>(p, s, eb, ee);
    case 64: return launch_bf16<64>(p, s, eb, ee);
    case 128: return launch_bf16<128>(p, s, eb, ee);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_bwd_f32(const BwdParams& p, hipStream_t s, hipEvent_t eb, hipEvent_t ee) {
  BwdParams q = p;
  q.dq_acc = nullptr;
  switch (p.D) {
    case 32: return launch_f32<32>(q, s, eb, ee);
    case 64: return launch_f32<64>(q, s, eb, ee);
    case 128: return launch_f32<128>(q, s, eb, ee);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
