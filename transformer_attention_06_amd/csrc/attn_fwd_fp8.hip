// Attention forward of fp8 (e4m3) operands for gfx950.
//
// The operands q, k, v are float8 e4m3 codes with one descale per tensor
// (tensorwise scaling, "nanochat Admin & Developer Guide", section 5
// "Precision: Explicit dtype & FP8"; the attention kernel takes fp8 as well
// as bf16 operands, section 6). The result is the attention of the
// dequantized operands:
//   s_ij = scale * dq * dk * <q8_i, k8_j>,  out_i = dv * sum_j p_ij v8_j,
// over the causal sliding window of the bf16 kernel; out is bf16, lse float32.
//
// Same structure as the bf16 kernel (128 queries per workgroup, 32 per
// wave, 64-key tiles through double-buffered LDS, S^T = K Q^T so that each
// lane owns one query), on the 32x32x64 fp8 MFMA (its scaled form with unit
// scales), which halves the products' share of a tile:
//   * S: A = 32 bytes of a K row from LDS, B = 32 bytes of the lane's q row
//     (registers); the contraction runs over d in 64-byte steps, both
//     operands taking byte e of lane half h from d = 32 h + e;
//   * P V: the probabilities are rounded to e4m3 and packed in the order the
//     accumulator holds them (byte e of lane half h <-> key
//     32 (e / 16) + 8 ((e % 16) / 4) + 4 h + e % 4 of the tile), which is
//     the B operand of O^T += V^T P^T. The matching A operand comes from four
//     8-row transpose reads (ds_read_b64_tr_b8: lane i of a 16-lane group
//     receives column i of 8 consecutive rows). Read q of half h must give
//     keys 16 q + 4 h + {0..3, 8..11}; the V tile is therefore stored with
//     bits 2 and 3 of its row index exchanged (LDS row r holds key
//     swap23(r)), a free choice of each copy lane's source row, so that
//     LDS rows 16 q + 8 h .. + 7 are exactly those keys.
// The row sum uses the float32 probabilities; only the P V product sees
// them rounded (relative error up to 2^-4).

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace nc {
namespace {

constexpr int F8_BM = 128;  // queries per workgroup
constexpr int F8_BN = 64;   // keys per tile
constexpr int F8_THREADS = 256;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0 / 0: both operands e4m3; E8M0 scale 127 = 1.0 for both
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)lds_addr);
}

// LDS row r of a V tile holds key swap23(r) (bits 2 and 3 exchanged).
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Chunk permutation of the V tile (chunk c of row r at c ^ swz_v(r)): the
// 32 lanes of a transpose read cover 8 consecutive rows x an aligned pair of
// chunks; the xor moves each row's pair to its own 32-byte bank slot (K
// tiles keep swz, which suits their 16-row operand reads).
template <int NC>
__device__ __forceinline__ int swz_v(int r) {
  return NC >= 8 ? ((r >> 1) & 3) << 1 : ((r >> 2) & 1) << 1;
}

template <int D>
__global__ __launch_bounds__(F8_THREADS, 3) void attn_fwd_fp8_kernel(Fp8FwdParams p) {
  constexpr int NC = D / 16;              // 16-byte chunks per row (one byte per element)
  constexpr int KS = D / 64;              // 64-wide steps of d in S
  constexpr int ND = D / 32;              // 32-row blocks of d in O^T
  constexpr int TILE = F8_BN * D;         // bytes of one K or V tile
  constexpr int RPI = 64 / NC;            // tile rows per copy instruction
  constexpr int IPW = F8_BN / RPI / 4;    // copy instructions per wave per tensor per tile
  static_assert(IPW >= 1 && KS >= 1, "tile/wave mismatch");
  __shared__ __attribute__((aligned(16))) unsigned char kv_lds[2][2][TILE];

  const int T = p.T;
  const int nqt = (T + F8_BM - 1) / F8_BM;
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
  const int t16 = lane & 15;

  const size_t qrs = (size_t)p.H * D;           // bytes between consecutive query rows
  const unsigned kvrs = (unsigned)(p.Hkv * D);  // bytes between consecutive key rows
  const unsigned char* qp = (const unsigned char*)p.q + (size_t)b * T * qrs + (size_t)h * D;
  const unsigned char* kp = (const unsigned char*)p.k + (size_t)b * T * kvrs + (size_t)g * D;
  const unsigned char* vp = (const unsigned char*)p.v + (size_t)b * T * kvrs + (size_t)g * D;
  const unsigned span = (unsigned)((size_t)(T - 1) * kvrs + D);
  const BufDesc krs = buf_desc(kp, span), vrs = buf_desc(vp, span);

  const bool full = p.window <= 0;
  const int win = p.window;
  const unsigned wlim = full ? 0x80000000u : (unsigned)win;
  auto tile_range = [&](int qt, int& first, int& last) {
    const int q0 = qt * F8_BM;
    first = (full ? 0 : max(0, q0 - win + 1)) / F8_BN;
    last = min(T - 1, q0 + F8_BM - 1) / F8_BN;
  };

  // Tile copies: lane l of instruction n writes LDS row (inst * RPI + l / NC),
  // physical chunk l % NC, holding logical chunk (l % NC) ^ swz(row) of its
  // source row (swz_v for V): the same row for K, key swap23(row) for V. Rows past the keys
  // present are clamped to T - 1 (finite, masked for every valid query).
  unsigned ld_k[IPW], ld_v[IPW];
  int ld_rk[IPW], ld_rv[IPW], ld_ck[IPW], ld_cv[IPW];
#pragma unroll
  for (int n = 0; n < IPW; ++n) {
    const int row = (wave * IPW + n) * RPI + lane / NC;
    ld_rk[n] = row;
    ld_rv[n] = swap23(row);
    ld_ck[n] = (lane % NC) ^ (swz<NC>(row) & (NC - 1));
    ld_cv[n] = (lane % NC) ^ (swz_v<NC>(row) & (NC - 1));
    ld_k[n] = (unsigned)(ld_rk[n] * kvrs + ld_ck[n] * 16);
    ld_v[n] = (unsigned)(ld_rv[n] * kvrs + ld_cv[n] * 16);
  }
  auto issue_tile = [&](int jt, int buf) {
    const int j0 = jt * F8_BN;
    if (j0 + F8_BN <= T) {
      const unsigned so = (unsigned)j0 * kvrs;
#pragma unroll
      for (int n = 0; n < IPW; ++n) {
        dma16(krs, ld_k[n], so, lds_u32(&kv_lds[buf][0][(wave * IPW + n) * RPI * D]));
        dma16(vrs, ld_v[n], so, lds_u32(&kv_lds[buf][1][(wave * IPW + n) * RPI * D]));
      }
    } else {
#pragma unroll
      for (int n = 0; n < IPW; ++n) {
        const unsigned ok = (unsigned)(min(j0 + ld_rk[n], T - 1) * kvrs + ld_ck[n] * 16);
        const unsigned ov = (unsigned)(min(j0 + ld_rv[n], T - 1) * kvrs + ld_cv[n] * 16);
        dma16(krs, ok, 0u, lds_u32(&kv_lds[buf][0][(wave * IPW + n) * RPI * D]));
        dma16(vrs, ov, 0u, lds_u32(&kv_lds[buf][1][(wave * IPW + n) * RPI * D]));
      }
    }
  };

  // Per-lane LDS byte offsets (tile-relative), fixed for the kernel:
  // K operand rows li (+32 for the second key block) at logical chunks
  // 4 ks + 2 hh and 4 ks + 2 hh + 1; V transpose reads of q at rows
  // 16 q + 8 hh + t16 / 2, byte 8 (t16 % 2) of logical chunk
  // 2 db + (li >= 16).
  int koff[KS][2], voff[ND][4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int lc = 4 * ks + 2 * hh + c;
      koff[ks][c] = li * D + ((lc ^ (swz<NC>(li) & (NC - 1))) << 4);
    }
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int row = 16 * qq + 8 * hh + (t16 >> 1);
      const int lc = 2 * db + (li >> 4);
      voff[db][qq] = row * D + ((lc ^ (swz_v<NC>(row) & (NC - 1))) << 4) + 8 * (t16 & 1);
    }

  int qw = 0, qi = 0;
  bool q_valid = false;
  int t_end = 0, next_first = -1;
  i32x8 qf[KS];  // the lane's q row as B operand bytes 64 ks + 32 hh + e
  float m2 = -INFINITY, lsum = 0.f;
  f32x16 o[ND];

  auto tile = [&](int jt, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmem();
    lds_barrier();
    if (jt < t_end)
      issue_tile(jt + 1, buf ^ 1);
    else if (next_first >= 0)
      issue_tile(next_first, buf ^ 1);
    const unsigned char* kl = kv_lds[buf][0];
    const unsigned char* vl = kv_lds[buf][1];

    const int j0 = jt * F8_BN;
    const bool any = (j0 <= qw + 31) && (full || j0 + F8_BN - 1 > qw - win);
    if (!any) return;
    const bool interior = (j0 + F8_BN - 1 <= qw) && (full || j0 > qw + 31 - win);

    f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const u32x4 a0 = *(const u32x4*)(kl + koff[ks][0] + jb * 32 * D);
        const u32x4 a1 = *(const u32x4*)(kl + koff[ks][1] + jb * 32 * D);
        const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        s[jb] = mfma_fp8(a, qf[ks], s[jb]);
      }
    // s[jb][r] = S[key j0 + 32 jb + 8 (r/4) + 4 hh + r%4][query qi] (unscaled)
    if (!interior) {
      const int base = qi - j0 - 4 * hh;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((unsigned)(base - (32 * jb + 8 * (r >> 2) + (r & 3))) >= wlim) s[jb][r] = -INFINITY;
    }
    float m4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      m4[c] = fmaxf(s[0][c], s[1][c]);
#pragma unroll
      for (int r = c + 4; r < 16; r += 4) m4[c] = fmaxf(fmaxf(m4[c], s[0][r]), s[1][r]);
    }
    const float mx = max_mod<32>(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    // the reference max moves only when the tile max exceeds it by more than
    // 8 (log2 units): the probabilities stay <= 256, inside e4m3's range
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

    // P as e4m3, packed in accumulator order: byte e <-> s[e / 16][e % 16]
    i32x8 pb;
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int jb = w >> 2, r0 = 4 * (w & 3);
      const float e0 = exp2_fast(fmaf(s[jb][r0], p.scale_log2, -m_use));
      const float e1 = exp2_fast(fmaf(s[jb][r0 + 1], p.scale_log2, -m_use));
      const float e2 = exp2_fast(fmaf(s[jb][r0 + 2], p.scale_log2, -m_use));
      const float e3 = exp2_fast(fmaf(s[jb][r0 + 3], p.scale_log2, -m_use));
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, wd, true);
      pb[w] = wd;
      rs0 += e0 + e2;
      rs1 += e1 + e3;
    }
    lsum += rs0 + rs1;

    // O^T += V^T P^T over the tile's 64 keys
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      i32x8 a;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const i32x2 x = lds_read_tr8(vl + voff[d][qq]);
        a[2 * qq] = x[0];
        a[2 * qq + 1] = x[1];
      }
      o[d] = mfma_fp8(a, pb, o[d]);
    }
  };

  auto run = [&](int qt, int t_begin, auto startc) __attribute__((always_inline)) {
    constexpr int S0 = decltype(startc)::value;
    const int qrow = qt * F8_BM + wave * 32 + li;
    qw = qt * F8_BM + wave * 32;
    qi = qrow;
    q_valid = qrow < T;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
      if (q_valid) {
        const unsigned char* src = qp + (size_t)qrow * qrs + 64 * ks + 32 * hh;
        w0 = *(const u32x4*)src;
        w1 = *(const u32x4*)(src + 16);
      }
      qf[ks] = (i32x8){(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
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
      const float inv = p.v_descale / lt;
      unsigned short* op = (unsigned short*)p.out + ((size_t)b * T + qrow) * p.H * D + (size_t)h * D;
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
  for (int i = 0; i < 2; ++i) {
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

}  // namespace

hipError_t launch_attn_fwd_fp8(const Fp8FwdParams& p, hipStream_t s) {
  const int nqt = (p.T + F8_BM - 1) / F8_BM;
  const dim3 grid((p.window <= 0 ? (nqt + 1) / 2 : nqt) * p.H * p.B), block(F8_THREADS);
  switch (p.D) {
    case 64: attn_fwd_fp8_kernel<64><<<grid, block, 0, s>>>(p); break;
    case 128: attn_fwd_fp8_kernel<128><<<grid, block, 0, s>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nc
