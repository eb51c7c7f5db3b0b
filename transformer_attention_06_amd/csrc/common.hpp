// Shared device/host helpers for the libncattn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nc {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// bf16 <-> f32. The float -> bf16 cast lowers to the hardware convert, which
// rounds to nearest even (checked on gfx950, including ties and subnormals).

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
  return __builtin_bit_cast(float, (unsigned)b << 16);
}
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(unsigned short, (bf16)f);
}
// Two floats -> one dword holding two bf16 (lo in bits 0..15).
__device__ __forceinline__ unsigned pack2_bf16(float lo, float hi) {
  return (unsigned)f32_to_bf16_bits(lo) | ((unsigned)f32_to_bf16_bits(hi) << 16);
}
// Unpack 8 bf16 held in a 16-byte vector into floats.
__device__ __forceinline__ void unpack8_bf16(u32x4 w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ u32x4 pack8_bf16(const float* f) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack2_bf16(f[2 * i], f[2 * i + 1]);
  return w;
}

// MFMA operand from 8 floats (element e of the operand = f[e]); packed
// two-at-a-time round-to-nearest-even conversions.
__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 a = __builtin_convertvector((f32x2){f[0], f[1]}, bf16x2);
  bf16x2 b = __builtin_convertvector((f32x2){f[2], f[3]}, bf16x2);
  bf16x2 c = __builtin_convertvector((f32x2){f[4], f[5]}, bf16x2);
  bf16x2 d = __builtin_convertvector((f32x2){f[6], f[7]}, bf16x2);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// Two floats -> one dword of two bf16 (lo first), one packed conversion.
__device__ __forceinline__ unsigned pk_bf16(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Raw buffer resource over [base, base + bytes) (no swizzle, no stride), for
// the buffer atomics.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// The same descriptor as four dwords (base address, stride 0, num_records,
// raw dword format), for the inline-assembly loads below.
typedef u32x4 BufDesc;
__device__ __forceinline__ BufDesc buf_desc(const void* base, unsigned bytes) {
  const unsigned long long a = (unsigned long long)(size_t)base;
  return (BufDesc){(unsigned)a, (unsigned)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
// LDS byte address of a pointer into __shared__ memory, wave-uniform.
__device__ __forceinline__ unsigned lds_u32(const void* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)p);
}
// Direct buffer -> LDS copies: lane l's 16 (dma16) or 4 (dma4) bytes at
// base + voffset + soffset land at lds + 16 l (4 l); lds is wave-uniform.
// They are written as inline assembly on purpose: the compiler then leaves
// them out of its bookkeeping of outstanding vector memory operations and
// inserts no waits for them (for the builtin it waits for every such copy
// in flight before any LDS read it cannot prove disjoint, which serialises
// a prefetch pipeline). Every reader of the destination must therefore wait
// for the copies itself (wait_vmcnt / wait_vmem_upto, which count them) and
// then synchronise the workgroup with lds_barrier().
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; nothing else here relies on its value
__device__ __forceinline__ void dma16(BufDesc d, unsigned voffset, unsigned soffset, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(d), "s"(soffset)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(BufDesc d, unsigned voffset, unsigned soffset, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(d), "s"(soffset)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// Workgroup barrier for LDS hand-offs: waits for this wave's own LDS
// operations, then s_barrier. It is a compiler memory barrier, but unlike
// __syncthreads it does not wait for outstanding vector memory operations
// (loads in flight, atomics), which is what lets prefetches overlap compute.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// sum of the two bf16 halves of w, plus c (v_dot2_f32_bf16 against (1, 1))
__device__ __forceinline__ float add2_bf16(unsigned w, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, c, false);
}

// Wait until all of this wave's global loads (including direct-to-LDS ones) completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// s_waitcnt with vmcnt = N (0..63) and no wait on the other counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}
// Wait until at most n (wave-uniform, clamped to 0..63) of this wave's vector
// memory operations are outstanding.
__device__ __forceinline__ void wait_vmem_upto(int n) {
#define NC_VMC_CASE(k) \
  case k:              \
    wait_vmcnt<k>();   \
    break;
  switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
    NC_VMC_CASE(0) NC_VMC_CASE(1) NC_VMC_CASE(2) NC_VMC_CASE(3) NC_VMC_CASE(4) NC_VMC_CASE(5) NC_VMC_CASE(6)
    NC_VMC_CASE(7) NC_VMC_CASE(8) NC_VMC_CASE(9) NC_VMC_CASE(10) NC_VMC_CASE(11) NC_VMC_CASE(12)
    NC_VMC_CASE(13) NC_VMC_CASE(14) NC_VMC_CASE(15) NC_VMC_CASE(16) NC_VMC_CASE(17) NC_VMC_CASE(18)
    NC_VMC_CASE(19) NC_VMC_CASE(20) NC_VMC_CASE(21) NC_VMC_CASE(22) NC_VMC_CASE(23) NC_VMC_CASE(24)
    NC_VMC_CASE(25) NC_VMC_CASE(26) NC_VMC_CASE(27) NC_VMC_CASE(28) NC_VMC_CASE(29) NC_VMC_CASE(30)
    NC_VMC_CASE(31) NC_VMC_CASE(32) NC_VMC_CASE(33) NC_VMC_CASE(34) NC_VMC_CASE(35) NC_VMC_CASE(36)
    NC_VMC_CASE(37) NC_VMC_CASE(38) NC_VMC_CASE(39) NC_VMC_CASE(40) NC_VMC_CASE(41) NC_VMC_CASE(42)
    NC_VMC_CASE(43) NC_VMC_CASE(44) NC_VMC_CASE(45) NC_VMC_CASE(46) NC_VMC_CASE(47) NC_VMC_CASE(48)
    NC_VMC_CASE(49) NC_VMC_CASE(50) NC_VMC_CASE(51) NC_VMC_CASE(52) NC_VMC_CASE(53) NC_VMC_CASE(54)
    NC_VMC_CASE(55) NC_VMC_CASE(56) NC_VMC_CASE(57) NC_VMC_CASE(58) NC_VMC_CASE(59) NC_VMC_CASE(60)
    NC_VMC_CASE(61) NC_VMC_CASE(62) default: wait_vmcnt<63>(); break;
  }
#undef NC_VMC_CASE
}
// Wait until at most n (rounded down to 0, 16 or 32; n wave-uniform) of this
// wave's vector memory operations are outstanding.
__device__ __forceinline__ void wait_vmem_leq(int n) {
  if (n >= 32)
    __builtin_amdgcn_s_waitcnt(0x8f70);  // vmcnt(32)
  else if (n >= 16)
    __builtin_amdgcn_s_waitcnt(0x4f70);  // vmcnt(16)
  else
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
}

// ---------------------------------------------------------------------------
// Exponentials: v_exp_f32 computes 2^x; callers fold log2(e) into their scale.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Sum over each aligned group of N lanes (N = 2, 4, 8 or 16), result in every
// lane of the group, with DPP moves inside 16-lane rows (no LDS traffic):
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group of 2..16 lanes");
  x += dpp_mov<0xB1>(x);                // quad_perm [1,0,3,2]
  if (N >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  if (N >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
  if (N >= 16) x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// Reductions over lanes with equal l % S (S = 4, 8, 16 or 32): every lane
// gets the sum (or maximum) over its class, with no LDS traffic. Inside a
// 16-lane row the partners come from DPP row rotations (x[i] + x[i - S] and
// so on, mod 16); across rows from v_permlane16_swap (rows 0<->1, 2<->3) and
// v_permlane32_swap (lanes l <-> l ^ 32). Either swap returns the pair of
// values in some order in its two results, so combining both results is
// symmetric and needs no lane select.
__device__ __forceinline__ unsigned f2u(float x) { return __builtin_bit_cast(unsigned, x); }
__device__ __forceinline__ float u2f(unsigned x) { return __builtin_bit_cast(float, x); }
template <bool MAX>
__device__ __forceinline__ float comb(float a, float b) { return MAX ? fmaxf(a, b) : a + b; }
template <int S, bool MAX>
__device__ __forceinline__ float reduce_mod(float x) {
  static_assert(S == 4 || S == 8 || S == 16 || S == 32, "lane class stride");
  if (S == 4) x = comb<MAX>(x, dpp_mov<0x124>(x));  // row_ror:4
  if (S <= 8) x = comb<MAX>(x, dpp_mov<0x128>(x));  // row_ror:8
  if (S <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    x = comb<MAX>(u2f(r[0]), u2f(r[1]));
  }
  const auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  return comb<MAX>(u2f(r[0]), u2f(r[1]));
}
template <int S>
__device__ __forceinline__ float sum_mod(float x) { return reduce_mod<S, false>(x); }
template <int S>
__device__ __forceinline__ float max_mod(float x) { return reduce_mod<S, true>(x); }

// ---------------------------------------------------------------------------
// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane t supplies the address of 4 consecutive 16-bit elements; the result
// of lane i holds, for e = 0..3, element (i % 4) of the 8 bytes addressed by
// lane 4e + i/4 of its group. So if lane t points at row (r0 + t/4), column
// (c0 + 4*(t%4)) of a row-major 16-bit matrix, lane i receives the column
// c0 + i of rows r0 .. r0+3.
// The pointer is cast to the LDS address space directly (not through an
// integer), so the compiler sees base + constant and folds the constant into
// the instruction's offset field instead of holding one address register per
// read.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)lds_addr);
}

__device__ __forceinline__ bf16x8 cat_bf16x8(s16x4 a, s16x4 b) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

// 32x32x16 bf16 MFMA, fp32 accumulate.
// Operand layouts (lane l, h = l / 32): A[m = l%32][k = 8h + e],
// B[k = 8h + e][n = l%32], e = 0..7. Result element r of lane l is
// C[8*(r/4) + 4h + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA, fp32 accumulate (lane l, t = l % 16, g = l / 16):
// A[m = t][k = 8g + e], B[k = 8g + e][n = t], e = 0..7; result element r of
// lane l is C[4g + r][t].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS tile layout: rows of NC 16-byte chunks (NC = elements per row / 8), no
// padding; chunk c of row r is stored at chunk position c ^ swz<NC>(r). The
// permutation makes both access patterns the kernels use conflict-free on
// the 64-bank LDS: 16 consecutive rows read at one logical chunk (MFMA
// operand rows, ds_read_b128) land on 16 distinct bank groups, and the
// 4 rows x 4 chunks read by 32 lanes of a transpose read do as well.
template <int NC>
__device__ __forceinline__ int swz(int r) {
  if (NC >= 16) return 4 * (r & 3) + ((r >> 2) & 3);
  if (NC == 8) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  return (r >> 2) & 3;
}
// Element offset of logical (row, col) in a swizzled tile with NC chunks per row.
template <int NC>
__device__ __forceinline__ int swz_off(int r, int col) {
  return r * (NC * 8) + ((((col >> 3) ^ swz<NC>(r)) & (NC - 1)) << 3) + (col & 7);
}

// The dK/dV kernel's q/dO tiles use another permutation: its operand reads
// are 16 consecutive rows at one chunk (ds_read_b128) and its transpose reads
// cover 4 rows x 4 aligned 8-byte pieces per 16 lanes (ds_read_b64_tr_b16).
// For 256-byte rows (NC = 16) the table below came out of a timed search
// over bit permutations of the row index with one xor fold: it runs the
// b128 pattern at the LDS peak (256 B/clk/CU, where a plain r & 15 xor also
// does) and the transpose pattern at 189 B/clk/CU (the row-major xor gets
// 128). As bits: chunk xor = (r3, r1, r2 ^ r3, r0 ^ r1). Rows of NC < 16
// chunks share a 256-byte bank window and keep a simpler interleave.
template <int NC>
__device__ __forceinline__ int swz_kv(int r) {
  if (NC >= 16)
    return ((r >> 3) & 1) | (r & 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 2) | (((r ^ (r >> 1)) & 1) << 3);
  if (NC == 8) return 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
  return 2 * ((r >> 2) & 1) + ((r >> 3) & 1);
}
template <int NC>
__device__ __forceinline__ int swz_kv_off(int r, int col) {
  return r * (NC * 8) + ((((col >> 3) ^ swz_kv<NC>(r)) & (NC - 1)) << 3) + (col & 7);
}

// Blocks -> XCD-contiguous logical ids. Workgroups are dealt to the 8 XCDs
// round-robin (block L runs on XCD L % 8); this maps the blocks that land on
// one XCD to one contiguous range of logical ids so that neighbouring work
// (the query tiles of one head) shares that XCD's L2.
__device__ __forceinline__ int xcd_remap(int L, int N) {
  const int q = N >> 3, r = N & 7;
  const int xcd = L & 7, pos = L >> 3;
  return xcd < r ? xcd * (q + 1) + pos : r * (q + 1) + (xcd - r) * q + pos;
}

}  // namespace nc
