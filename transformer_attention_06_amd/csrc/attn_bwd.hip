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
//   pre:  delta_i = <dout_i, out_i> in float32; clear the float32 dq accumulator.
//   main: one workgroup per (b, kv head, 128-key tile); each of the 4 waves
//         keeps 32 keys' K and V fragments in registers and accumulates dK^T
//         and dV^T for them over every query head of the GQA group and every
//         64-query tile that intersects the band. S = Q K^T and dP = dO V^T
//         come out with one key column per lane, which is directly the
//         B-operand layout of dV^T += dO^T P and dK^T += Q^T dS; dO^T and
//         Q^T are LDS transpose reads. dS goes through LDS once so that
//         dQ = dS K for the 128 keys is formed per workgroup and added to
//         the float32 accumulator with one atomic per element.
//   post: dq = bf16(scale-applied accumulator).
// f32 path: plain per-key (dk, dv) and per-query (dq) loops in float32.

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace nc {
namespace {

constexpr int BWD_BN = 128;  // keys per workgroup (32 per wave)
constexpr int BWD_BM = 64;   // queries per step
constexpr int BWD_THREADS = 256;

// --------------------------------------------------------------------------
// delta = rowsum(dout * out) (float32), and dq_acc := 0 when present.
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
    // row = (b * T + t) * H + h  ->  delta[b, h, t]
    const long bt = row / p.H;
    const int h = (int)(row - bt * p.H);
    const long b = bt / p.T;
    const int t = (int)(bt - b * p.T);
    p.delta[((size_t)b * p.H + h) * p.T + t] = acc;
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
  constexpr int QLOADS = BWD_BM * NC / BWD_THREADS;
  constexpr int KLOADS = BWD_BN * NC / BWD_THREADS;
  static_assert(QLOADS >= 1 && KLOADS >= 1, "tile/thread mismatch");
  __shared__ __attribute__((aligned(16))) unsigned short k_lds[BWD_BN * D];
  __shared__ __attribute__((aligned(16))) unsigned short q_lds[BWD_BM * D];
  __shared__ __attribute__((aligned(16))) unsigned short do_lds[BWD_BM * D];
  __shared__ __attribute__((aligned(16))) unsigned short ds_lds[BWD_BN * BWD_BM];
  __shared__ float lse2_lds[BWD_BM];
  __shared__ float delta_lds[BWD_BM];

  const int T = p.T;
  const int nkt = (T + BWD_BN - 1) / BWD_BN;
  const int N = nkt * p.Hkv * p.B;
  const int logical = xcd_remap(blockIdx.x, N);
  const int bg = logical / nkt;
  const int kt = logical - bg * nkt;  // early key tiles (most queries) first
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int G = p.H / p.Hkv;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hh = lane >> 5;
  const int grp = lane >> 4, t16 = lane & 15;
  const int j0 = kt * BWD_BN;
  const int kw = j0 + wave * 32;
  const int kj = kw + li;  // this lane's key

  const size_t qrs = (size_t)p.H * D;
  const size_t kvrs = (size_t)p.Hkv * D;
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)b * T * kvrs + (size_t)g * D;
  const unsigned short* vp = (const unsigned short*)p.v + (size_t)b * T * kvrs + (size_t)g * D;

  // K tile -> LDS (B operand of dQ = dS K via transpose reads).
#pragma unroll
  for (int n = 0; n < KLOADS; ++n) {
    const int c = tid + n * BWD_THREADS;
    const int row = c / NC, ch = c - row * NC;
    const int j = j0 + row;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (j < T) w = *(const u32x4*)(kp + (size_t)j * kvrs + ch * 8);
    *(u32x4*)(k_lds + swz_off<NC>(row, ch * 8)) = w;
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

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    dk[d] = (f32x16){};
    dv[d] = (f32x16){};
  }

  const bool full = p.window <= 0;
  const int win = p.window;
  const int i_last = full ? T - 1 : min(T - 1, j0 + BWD_BN - 1 + win - 1);
  const int it_begin = j0 / BWD_BM, n_it = i_last / BWD_BM - it_begin + 1;
  const int n_steps = G * n_it;
  const int tr_row = t16 >> 2;
  const int tr_col = 16 * (grp & 1) + 4 * (t16 & 3);

  // Registers holding the next step's q/dO tile rows, lse and delta.
  u32x4 qreg[QLOADS], oreg[QLOADS];
  float lreg = INFINITY, dreg = 0.f;
  auto prefetch = [&](int step) {
    const int hq = step / n_it;
    const int i0 = (it_begin + step - hq * n_it) * BWD_BM;
    const int h = g * G + hq;
    const unsigned short* qp = (const unsigned short*)p.q + (size_t)b * T * qrs + (size_t)h * D;
    const unsigned short* dop = (const unsigned short*)p.dout + (size_t)b * T * qrs + (size_t)h * D;
#pragma unroll
    for (int n = 0; n < QLOADS; ++n) {
      const int c = tid + n * BWD_THREADS;
      const int row = c / NC, ch = c - row * NC;
      const int i = i0 + row;
      qreg[n] = (u32x4){0u, 0u, 0u, 0u};
      oreg[n] = (u32x4){0u, 0u, 0u, 0u};
      if (i < T) {
        qreg[n] = *(const u32x4*)(qp + (size_t)i * qrs + ch * 8);
        oreg[n] = *(const u32x4*)(dop + (size_t)i * qrs + ch * 8);
      }
    }
    if (tid < BWD_BM) {
      const int i = i0 + tid;
      const size_t li2 = ((size_t)b * p.H + h) * T + i;
      lreg = i < T ? p.lse[li2] * kLog2e : INFINITY;
      dreg = i < T ? p.delta[li2] : 0.f;
    }
  };

  prefetch(0);
  for (int step = 0; step < n_steps; ++step) {
    const int hq = step / n_it;
    const int i0 = (it_begin + step - hq * n_it) * BWD_BM;
    const int h = g * G + hq;
    __syncthreads();  // every reader of the previous step's tiles is done
#pragma unroll
    for (int n = 0; n < QLOADS; ++n) {
      const int c = tid + n * BWD_THREADS;
      const int row = c / NC, ch = c - row * NC;
      *(u32x4*)(q_lds + swz_off<NC>(row, ch * 8)) = qreg[n];
      *(u32x4*)(do_lds + swz_off<NC>(row, ch * 8)) = oreg[n];
    }
    if (tid < BWD_BM) {
      lse2_lds[tid] = lreg;
      delta_lds[tid] = dreg;
    }
    __syncthreads();
    if (step + 1 < n_steps) prefetch(step + 1);

    const bool any = (kw <= i0 + BWD_BM - 1) && (full || kw + 31 > i0 - win);
    const bool interior = (kw + 31 <= i0) && (full || kw > i0 + BWD_BM - 1 - win);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      float dsr[16];
      if (any) {
        f32x16 sacc = (f32x16){}, dpacc = (f32x16){};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const bf16x8 aq = *(const bf16x8*)(q_lds + swz_off<NC>(32 * ib + li, 16 * st + 8 * hh));
          sacc = mfma32(aq, kf[st], sacc);
          const bf16x8 ad = *(const bf16x8*)(do_lds + swz_off<NC>(32 * ib + li, 16 * st + 8 * hh));
          dpacc = mfma32(ad, vf[st], dpacc);
        }
        // sacc[r] = S[query i0 + 32 ib + 8 (r/4) + 4 hh + r%4][key kj]
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int il = 32 * ib + 8 * (r >> 2) + 4 * hh + (r & 3);
          float pv = exp2_fast(fmaf(sacc[r], p.scale_log2, -lse2_lds[il]));
          if (!interior) {
            const int i = i0 + il;
            const bool vis = (kj <= i) && (full || kj > i - win);
            if (!vis) pv = 0.f;
          }
          pr[r] = pv;
          dsr[r] = pv * (dpacc[r] - delta_lds[il]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS over these 32 queries.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 pb = to_bf16x8(&pr[8 * u]);
          const bf16x8 sb = to_bf16x8(&dsr[8 * u]);
          const int r1 = 32 * ib + 16 * u + 4 * hh + tr_row;
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const int col = 32 * d + tr_col;
            const s16x4 o1 = lds_read_tr16(do_lds + swz_off<NC>(r1, col));
            const s16x4 o2 = lds_read_tr16(do_lds + swz_off<NC>(r1 + 8, col));
            dv[d] = mfma32(cat_bf16x8(o1, o2), pb, dv[d]);
            const s16x4 q1 = lds_read_tr16(q_lds + swz_off<NC>(r1, col));
            const s16x4 q2 = lds_read_tr16(q_lds + swz_off<NC>(r1 + 8, col));
            dk[d] = mfma32(cat_bf16x8(q1, q2), sb, dk[d]);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) dsr[r] = 0.f;
      }
      // dS^T -> LDS: row = key (wave*32 + li), 4 consecutive queries per store.
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 w;
        w[0] = pack2_bf16(dsr[4 * rg], dsr[4 * rg + 1]);
        w[1] = pack2_bf16(dsr[4 * rg + 2], dsr[4 * rg + 3]);
        *(u32x2*)(ds_lds + swz_off<NCS>(wave * 32 + li, 32 * ib + 8 * rg + 4 * hh)) = w;
      }
    }
    __syncthreads();

    // dQ[i][d] = sum over the 128 keys of dS[i][j] K[j][d]; output blocks
    // (ib, db) are dealt to the waves.
    float* dqa = p.dq_acc + (size_t)b * T * qrs + (size_t)h * D;
    for (int n = wave; n < 2 * ND; n += 4) {
      const int ib = n / ND, db = n - (n / ND) * ND;
      f32x16 acc = (f32x16){};
#pragma unroll
      for (int u = 0; u < BWD_BN / 16; ++u) {
        const int r0 = 16 * u + 8 * hh + tr_row;
        const s16x4 a1 = lds_read_tr16(ds_lds + swz_off<NCS>(r0, 32 * ib + tr_col));
        const s16x4 a2 = lds_read_tr16(ds_lds + swz_off<NCS>(r0 + 4, 32 * ib + tr_col));
        const s16x4 b1 = lds_read_tr16(k_lds + swz_off<NC>(r0, 32 * db + tr_col));
        const s16x4 b2 = lds_read_tr16(k_lds + swz_off<NC>(r0 + 4, 32 * db + tr_col));
        acc = mfma32(cat_bf16x8(a1, a2), cat_bf16x8(b1, b2), acc);
      }
      // acc[r] = dQ[query i0 + 32 ib + 8 (r/4) + 4 hh + r%4][d = 32 db + li]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 32 * ib + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (i < T) atomicAdd(dqa + (size_t)i * qrs + 32 * db + li, acc[r] * p.scale);
      }
    }
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
        wk[0] = pack2_bf16(dk[d][4 * rg] * p.scale, dk[d][4 * rg + 1] * p.scale);
        wk[1] = pack2_bf16(dk[d][4 * rg + 2] * p.scale, dk[d][4 * rg + 3] * p.scale);
        wv[0] = pack2_bf16(dv[d][4 * rg], dv[d][4 * rg + 1]);
        wv[1] = pack2_bf16(dv[d][4 * rg + 2], dv[d][4 * rg + 3]);
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
