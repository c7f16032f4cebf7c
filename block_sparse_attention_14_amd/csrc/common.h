// Device helpers shared by the gfx950 kernels: vector types, bf16 plumbing,
// the 16x16x32 bf16 MFMA and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sol {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 64;  // Bq = Bk = 64 tokens per block

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float pair -> packed bf16, one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16] and
// holds D[4*(l/16) + e][l%16], e = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Cross-lane moves inside a row of 16 lanes (DPP, a VALU operand modifier;
// no LDS round trip). Controls: quad_perm [1,0,3,2] swaps neighbours,
// row_ror:8 rotates a row by 8.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppRor8 = 0x128;  // row_ror:8, lane i of a row of 16 reads lane i ^ 8

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 16-byte load; bytes at or beyond the resource's size read as zero.
__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 ld16f(rsrc_t r, uint32_t voff, uint32_t soff) {
  const uint4 u = ld16(r, voff, soff);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

// Sum of a value over the lanes of a wave that share lane % CH (CH = 8 or
// 16): one DPP step for lane ^ 8 when CH = 8, then permlane swaps for
// lane ^ 16 and lane ^ 32. Every lane of a group ends with the same sum.
template <int CH>
__device__ __forceinline__ float colsum_rows(float x) {
  if (CH == 8) x += dpp<kDppRor8>(x);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace sol
