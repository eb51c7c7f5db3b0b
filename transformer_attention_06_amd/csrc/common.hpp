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

// MFMA operand from 8 floats (element e of the operand = f[e]).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  return __builtin_bit_cast(bf16x8, pack8_bf16(f));
}

// ---------------------------------------------------------------------------
// Exponentials: v_exp_f32 computes 2^x; callers fold log2(e) into their scale.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

// ---------------------------------------------------------------------------
// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane t supplies the address of 4 consecutive 16-bit elements; the result
// of lane i holds, for e = 0..3, element (i % 4) of the 8 bytes addressed by
// lane 4e + i/4 of its group. So if lane t points at row (r0 + t/4), column
// (c0 + 4*(t%4)) of a row-major 16-bit matrix, lane i receives the column
// c0 + i of rows r0 .. r0+3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)(
          (size_t)lds_addr)));
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
