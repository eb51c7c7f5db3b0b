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
//   * K/V tiles of 64 keys copied by buffer-to-LDS loads straight into a
//     double-buffered, XOR-swizzled LDS tile, the next tile in flight while
//     the current one is consumed; all LDS addresses are per-lane constants
//     plus immediates (the loop is unrolled over the two buffers);
//   * S^T = K Q^T on 32x32x16 bf16 MFMA, so that each lane owns one query
//     column: the row max and row sum need no cross-lane reduction except
//     one exchange between the two half-waves;
//   * the exponentiated scores come straight out of the accumulator in the
//     B-operand layout of O^T += V^T P^T (the contraction index is permuted
//     identically on both operands), and V^T is read with LDS transpose
//     reads;
//   * the running max only moves when a tile exceeds it by more than a
//     factor 2^8, so the O rescale is rare;
//   * tiles entirely outside the causal band or window are never visited;
//     element masks are applied only on tiles that cut the band's edges.
// Both kernels also take a chunk of queries against a KV cache (the SDPA
// fallback's chunked-inference case, "nanochat Admin & Developer Guide",
// section 6): chunk row t of batch row b sits at position q_off[b] + t and
// the band is shifted by q_off[b]; keys are read from the cache rows.
// The bf16 kernel can also take raw queries and apply the QK prologue to each
// row as it loads it (section 3: weightless RMSNorm, then half-split RoPE),
// storing q' for the backward; the keys then come from a k-only prologue.
// f32 kernel: plain per-query loop in float32, for the fp32 configurations.

#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace nc {
namespace {

constexpr int FWD_BM = 128;  // queries per workgroup
constexpr int FWD_BN = 64;   // keys per tile
constexpr int FWD_THREADS = 256;

template <int D, bool PRO>
__global__ __launch_bounds__(FWD_THREADS, 2) void attn_fwd_bf16_kernel(FwdParams p) {
  constexpr int NC = D / 8;  // 16-byte chunks per row (LDS tiles are swizzled, unpadded)
  constexpr int NS = D / 16;
  constexpr int ND = D / 32;
  constexpr int TILE = FWD_BN * D;        // elements of one K or V tile
  constexpr int RPI = 64 / NC;            // tile rows per direct-to-LDS instruction (64 lanes x 16 B)
  constexpr int IPW = FWD_BN / RPI / 4;   // such instructions per wave per tensor per tile
  static_assert(IPW >= 1 && FWD_BN % (4 * RPI) == 0, "tile/wave mismatch");
  // [buffer][K or V][tile]: the next tile streams into one buffer while the other is read
  __shared__ __attribute__((aligned(16))) unsigned short kv_lds[2][2][TILE];

  // Under the full causal mask a workgroup takes query tiles nqt-1-r and r
  // of one (b, h), in that order: their key counts add up to the same for
  // every r, so the workgroups are of equal weight and the grid has no tail
  // of heavy late tiles; the first K/V tile of the second query tile is
  // loaded while the first one finishes. Under a window the per-tile work
  // is nearly flat already: one query tile per workgroup, late tiles first.
  const int T = p.T;
  const int nqt = (T + FWD_BM - 1) / FWD_BM;
  const bool paired = p.window <= 0;
  const int nunit = paired ? (nqt + 1) / 2 : nqt;
  const int N = nunit * p.H * p.B;
  const int logical = xcd_remap(blockIdx.x, N);
  const int bh = logical / nunit;
  const int r_pair = logical - bh * nunit;
  const int b = bh / p.H, h = bh - b * p.H;
  const int g = h / (p.H / p.Hkv);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int li = lane & 31, hh = lane >> 5;
  const int grp = lane >> 4, t16 = lane & 15;

  const size_t qrs = (size_t)p.H * D;
  // position of chunk row 0 (0 without a cache) and the keys present
  const int off = p.q_off ? __builtin_amdgcn_readfirstlane(p.q_off[b]) : 0;
  const int Tk = off + T;
  if (off < 0 || Tk > p.T_kv) {  // a cache length the host could not check: NaN rows
    const int qt_a = nqt - 1 - r_pair, qt_b = r_pair;
    for (int pass = 0; pass < (paired && qt_b < qt_a ? 2 : 1); ++pass) {
      const int q0 = (pass == 0 ? qt_a : qt_b) * FWD_BM;
      for (int i = tid; i < FWD_BM * (D / 8); i += FWD_THREADS) {
        const int r = q0 + i / (D / 8);
        if (r < T)
          *(u32x4*)((unsigned short*)p.out + ((size_t)b * T + r) * qrs + (size_t)h * D + (i % (D / 8)) * 8) =
              (u32x4){0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
      }
      if (tid < FWD_BM && q0 + tid < T) p.lse[((size_t)b * p.H + h) * T + q0 + tid] = NAN;
    }
    return;
  }
  const unsigned kvrs = (unsigned)(p.Hkv * D);  // elements between consecutive positions
  // RoPE position of query row 0 (query prologue only)
  const int pos0 = PRO && p.pos_offset ? __builtin_amdgcn_readfirstlane(p.pos_offset[b]) : 0;
  const unsigned short* qp = (const unsigned short*)p.q + (size_t)b * T * qrs + (size_t)h * D;
  const unsigned short* kp = (const unsigned short*)p.k + (size_t)b * p.T_kv * kvrs + (size_t)g * D;
  const unsigned short* vp = (const unsigned short*)p.v + (size_t)b * p.T_kv * kvrs + (size_t)g * D;
  // this (b, g)'s key rows 0 .. Tk-1 span (Tk - 1) * kvrs + D elements
  const unsigned span = (unsigned)(((size_t)(Tk - 1) * kvrs + D) * 2);
  const BufDesc krs = buf_desc(kp, span), vrs = buf_desc(vp, span);

  const bool full = p.window <= 0;
  const int win = p.window;
  // key j is visible to query i iff (unsigned)(i - j) < wlim
  const unsigned wlim = full ? 0x80000000u : (unsigned)win;
  // key tiles [first, last] of query tile qt
  auto tile_range = [&](int qt, int& first, int& last) {
    const int q0 = off + qt * FWD_BM;  // position of the tile's first query
    first = (full ? 0 : max(0, q0 - win + 1)) / FWD_BN;
    last = min(Tk - 1, q0 + FWD_BM - 1) / FWD_BN;
  };

  // Tile loads: lane l of instruction n writes tile row (inst*RPI + l/NC),
  // physical chunk l%NC, which holds logical chunk (l%NC) ^ swz(row). The
  // lane's source offset inside the tile is fixed; the tile and instruction
  // offsets are uniform. The last tile may run past the keys present: its
  // rows are clamped to Tk-1 (finite data, masked for every valid query).
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
    const int j0 = jt * FWD_BN;
    if (j0 + FWD_BN <= Tk) {
      const unsigned so = (unsigned)j0 * kvrs * 2u;
#pragma unroll
      for (int n = 0; n < IPW; ++n) {
        dma16(krs, ld_off[n], so, lds_u32(&kv_lds[buf][0][(wave * IPW + n) * RPI * D]));
        dma16(vrs, ld_off[n], so, lds_u32(&kv_lds[buf][1][(wave * IPW + n) * RPI * D]));
      }
    } else {
#pragma unroll
      for (int n = 0; n < IPW; ++n) {
        const int j = min(j0 + ld_row[n], Tk - 1);
        const unsigned vo = (unsigned)(j * kvrs + ld_ch[n] * 8) * 2u;
        dma16(krs, vo, 0u, lds_u32(&kv_lds[buf][0][(wave * IPW + n) * RPI * D]));
        dma16(vrs, vo, 0u, lds_u32(&kv_lds[buf][1][(wave * IPW + n) * RPI * D]));
      }
    }
  };

  // Per-lane LDS element offsets (tile-relative), fixed for the whole kernel:
  // K operand rows li (+32 for the second key block) at chunk 2 st + hh;
  // V^T transpose reads at rows 4 hh + t16/4 (+8) (+16 u + 32 jb), columns
  // 32 d + 16 (grp & 1) + 4 (t16 & 3).
  int koff[NS], voff1[ND], voff2[ND];
#pragma unroll
  for (int st = 0; st < NS; ++st) koff[st] = swz_off<NC>(li, 16 * st + 8 * hh);
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    const int col = 32 * d + 16 * (grp & 1) + 4 * (t16 & 3);
    voff1[d] = swz_off<NC>(4 * hh + (t16 >> 2), col);
    voff2[d] = swz_off<NC>(4 * hh + (t16 >> 2) + 8, col);
  }

  // state of the query tile being processed
  int qw = 0, qi = 0;    // positions of this wave's first query and of this lane's query
  bool q_valid = false;
  int t_end = 0;         // its last key tile
  int next_first = -1;   // first key tile of the next query tile (-1: none)
  bf16x8 qf[NS];         // q as the B operand of S^T = K Q^T: q[qi][16 s + 8 hh + e]
  float m2 = -INFINITY;  // running reference max (log2 units) for this query
  float lsum = 0.f;      // running sum over this lane's half of the keys
  f32x16 o[ND];

  auto tile = [&](int jt, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmem();      // this wave's copies of tile jt (the only loads in flight)
    lds_barrier();    // everyone's copies of tile jt landed; the other buffer is free
    if (jt < t_end)
      issue_tile(jt + 1, buf ^ 1);
    else if (next_first >= 0)
      issue_tile(next_first, buf ^ 1);
    const unsigned short* kl = kv_lds[buf][0];
    const unsigned short* vl = kv_lds[buf][1];

    const int j0 = jt * FWD_BN;
    const bool any = (j0 <= qw + 31) && (full || j0 + FWD_BN - 1 > qw - win);
    if (!any) return;
    const bool interior = (j0 + FWD_BN - 1 <= qw) && (full || j0 > qw + 31 - win);

    f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const bf16x8 a = *(const bf16x8*)(kl + koff[st] + jb * 32 * D);
        s[jb] = mfma32(a, qf[st], s[jb]);
      }
    // s[jb][r] = S[key j0 + 32 jb + 8 (r/4) + 4 hh + r%4][query qi]
    if (!interior) {
      const int base = qi - j0 - 4 * hh;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((unsigned)(base - (32 * jb + 8 * (r >> 2) + (r & 3))) >= wlim) s[jb][r] = -INFINITY;
    }
    // tile max of this query: four independent chains, then the two half-waves
    float m4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      m4[c] = fmaxf(s[0][c], s[1][c]);
#pragma unroll
      for (int r = c + 4; r < 16; r += 4) m4[c] = fmaxf(fmaxf(m4[c], s[0][r]), s[1][r]);
    }
    const float mx = max_mod<32>(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    // The reference max only moves up when the tile max exceeds it by more than
    // 8 (a factor 2^8): the exponentials stay <= 256 and O is rescaled rarely.
    const float mt = mx * p.scale_log2;
    const bool raise = mt > m2 + 8.f;
    float alpha = 1.f;
    if (raise) {
      alpha = exp2_fast(m2 - mt);
      m2 = mt;
    }
    if (__any(raise)) {
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      lsum *= alpha;
    }
    const float m_use = (m2 == -INFINITY) ? 0.f : m2;

    // P^T as bf16 B operands (8 per 16 keys); row sums of the float values.
    unsigned pw[2][8];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = exp2_fast(fmaf(s[jb][r], p.scale_log2, -m_use));
        const float e1 = exp2_fast(fmaf(s[jb][r + 1], p.scale_log2, -m_use));
        pw[jb][r >> 1] = pk_bf16(e0, e1);
        rs0 += e0;
        rs1 += e1;
      }
    lsum += rs0 + rs1;

    // O^T += V^T P^T over the tile's 64 keys.
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 pq = {pw[jb][4 * u], pw[jb][4 * u + 1], pw[jb][4 * u + 2], pw[jb][4 * u + 3]};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pq);
        const int rb = (32 * jb + 16 * u) * D;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const s16x4 x1 = lds_read_tr16(vl + voff1[d] + rb);
          const s16x4 x2 = lds_read_tr16(vl + voff2[d] + rb);
          o[d] = mfma32(cat_bf16x8(x1, x2), pb, o[d]);
        }
      }
  };

  auto run = [&](int qt, int t_begin, auto startc) __attribute__((always_inline)) {
    constexpr int S0 = decltype(startc)::value;  // buffer of the first key tile
    const int qrow = qt * FWD_BM + wave * 32 + li;  // this lane's query row of q / out
    qw = off + qt * FWD_BM + wave * 32;
    qi = qw + li;
    q_valid = qrow < T;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (q_valid) w = *(const u32x4*)(qp + (size_t)qrow * qrs + 16 * s + 8 * hh);
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
    // query prologue: the lane's cos/sin rows are requested right after q
    const int pos = qrow + pos0;
    const bool pos_ok = pos >= 0 && pos < p.T_rope;
    f32x4 cv[PRO ? NS / 2 : 1][2], sv[PRO ? NS / 2 : 1][2];
    if constexpr (PRO) {
      const size_t toff = (size_t)((q_valid && pos_ok) ? pos : 0) * (D / 2) + 8 * hh;
#pragma unroll
      for (int s = 0; s < NS / 2; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          cv[s][i] = *(const f32x4*)(p.cos_tab + toff + 16 * s + 4 * i);
          sv[s][i] = *(const f32x4*)(p.sin_tab + toff + 16 * s + 4 * i);
        }
    }
    if constexpr (PRO) {
      // RMSNorm + RoPE of this lane's query row in the operand layout: the lane
      // holds elements 16 s + 8 hh + e, and element d < D/2 pairs with
      // d + D/2, held by the same lane at s + NS/2. The sum of squares adds
      // the two half-waves' shares, taken straight from the packed row. q' is
      // rounded to bf16, used and stored.
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 w = __builtin_bit_cast(u32x4, qf[s]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __builtin_bit_cast(float, w[i] << 16), hi = __builtin_bit_cast(float, w[i] & 0xffff0000u);
          ss = fmaf(lo, lo, fmaf(hi, hi, ss));
        }
      }
      ss = sum_mod<32>(ss);
      const float inv_r = 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
      unsigned short* qo = (unsigned short*)p.q_out + ((size_t)b * T + qrow) * qrs + (size_t)h * D;
#pragma unroll
      for (int s = 0; s < NS / 2; ++s) {
        float xl[8], xh[8];
        unpack8_bf16(__builtin_bit_cast(u32x4, qf[s]), xl);
        unpack8_bf16(__builtin_bit_cast(u32x4, qf[s + NS / 2]), xh);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float cs = cv[s][e >> 2][e & 3], sn = sv[s][e >> 2][e & 3];
          const float a = xl[e] * inv_r, bb = xh[e] * inv_r;
          xl[e] = pos_ok ? fmaf(a, cs, -bb * sn) : NAN;
          xh[e] = pos_ok ? fmaf(a, sn, bb * cs) : NAN;
        }
        const u32x4 wl = pack8_bf16(xl), wh = pack8_bf16(xh);
        qf[s] = __builtin_bit_cast(bf16x8, wl);
        qf[s + NS / 2] = __builtin_bit_cast(bf16x8, wh);
        if (q_valid) {
          *(u32x4*)(qo + 16 * s + 8 * hh) = wl;
          *(u32x4*)(qo + 16 * (s + NS / 2) + 8 * hh) = wh;
        }
      }
    }
    m2 = -INFINITY;
    lsum = 0.f;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = (f32x16){};
    for (int jt = t_begin; jt <= t_end; jt += 2) {
      tile(jt, std::integral_constant<int, S0>{});
      if (jt + 1 <= t_end) tile(jt + 1, std::integral_constant<int, S0 ^ 1>{});
    }

    const float lt = sum_mod<32>(lsum);
    if (q_valid) {
      const float inv = 1.f / lt;
      unsigned short* op = (unsigned short*)p.out + ((size_t)b * T + qrow) * qrs + (size_t)h * D;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          u32x2 w;
          w[0] = pk_bf16(o[d][4 * rg] * inv, o[d][4 * rg + 1] * inv);
          w[1] = pk_bf16(o[d][4 * rg + 2] * inv, o[d][4 * rg + 3] * inv);
          *(u32x2*)(op + 32 * d + 8 * rg + 4 * hh) = w;
        }
      if (hh == 0) p.lse[((size_t)b * p.H + h) * T + qrow] = (m2 + __builtin_log2f(lt)) * kLn2;
    }
  };

  const int qt_a = nqt - 1 - r_pair, qt_b = r_pair;
  const int n_pass = paired && qt_b < qt_a ? 2 : 1;
  int first[2], last[2];
  tile_range(qt_a, first[0], last[0]);
  tile_range(qt_b, first[1], last[1]);
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // uniform by construction; said so for the copies' scalar operands
    first[i] = __builtin_amdgcn_readfirstlane(first[i]);
    last[i] = __builtin_amdgcn_readfirstlane(last[i]);
  }
  issue_tile(first[0], 0);
  int start = 0;
  for (int pass = 0; pass < n_pass; ++pass) {
    t_end = last[pass];
    next_first = pass + 1 < n_pass ? first[pass + 1] : -1;
    if (start == 0)
      run(pass == 0 ? qt_a : qt_b, first[pass], std::integral_constant<int, 0>{});
    else
      run(pass == 0 ? qt_a : qt_b, first[pass], std::integral_constant<int, 1>{});
    start = (start + last[pass] - first[pass] + 1) & 1;
  }
}

// ---------------------------------------------------------------------------
// float32: one thread per query, online softmax over its visible keys.
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(FwdParams p) {
  const int T = p.T;
  const int qr_ = blockIdx.x * 64 + threadIdx.x;  // query row of q / out
  const int h = blockIdx.y, b = blockIdx.z;
  if (qr_ >= T) return;
  const int off = p.q_off ? p.q_off[b] : 0;
  float* o = (float*)p.out + (((size_t)b * T + qr_) * p.H + h) * D;
  if (off < 0 || off + T > p.T_kv) {  // a cache length the host could not check: NaN row
    for (int d = 0; d < D; ++d) o[d] = NAN;
    p.lse[((size_t)b * p.H + h) * T + qr_] = NAN;
    return;
  }
  const int qi = off + qr_;  // position
  const int g = h / (p.H / p.Hkv);
  const float* q = (const float*)p.q + (((size_t)b * T + qr_) * p.H + h) * D;
  const float* kb = (const float*)p.k + ((size_t)b * p.T_kv * p.Hkv + g) * D;
  const float* vb = (const float*)p.v + ((size_t)b * p.T_kv * p.Hkv + g) * D;
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
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = acc[d] * inv;
  p.lse[((size_t)b * p.H + h) * T + qr_] = m + logf(l);
}


template <bool PRO>
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s) {
  const int nqt = (p.T + FWD_BM - 1) / FWD_BM;
  const dim3 grid((p.window <= 0 ? (nqt + 1) / 2 : nqt) * p.H * p.B), block(FWD_THREADS);
  switch (p.D) {
    case 32: attn_fwd_bf16_kernel<32, PRO><<<grid, block, 0, s>>>(p); break;
    case 64: attn_fwd_bf16_kernel<64, PRO><<<grid, block, 0, s>>>(p); break;
    case 128: attn_fwd_bf16_kernel<128, PRO><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdParams& p, hipStream_t s) {
  return p.q_out ? launch_fwd_bf16<true>(p, s) : launch_fwd_bf16<false>(p, s);
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
