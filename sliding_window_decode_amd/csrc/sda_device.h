// sda_device.h -- gfx950 device helpers shared by the decode-attention kernels: vector types,
// exact fp8/fp4 -> bf16 conversions, LDS transpose reads, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef const __attribute__((address_space(1))) u32x4 gbl_u32x4;
typedef const __attribute__((address_space(1))) uint32_t gbl_u32;
typedef const __attribute__((address_space(1))) uint16_t gbl_u16;

__device__ __forceinline__ u32x4 ld_global_16(uint64_t addr) { return *(gbl_u32x4*)addr; }
__device__ __forceinline__ uint32_t ld_global_u16(uint64_t addr) { return *(gbl_u16*)addr; }

// Exact e4m3fn -> bf16 of the 4 codes of a word (the gfx950 conversion decodes the OCP format; every
// e4m3 value has at most 4 significant bits, so the bf16 result is exact).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) { return __builtin_amdgcn_cvt_pk_f32_fp8(byte, false)[0]; }

// Two e2m1 codes of byte `SEL` of w (low nibble first) times an e4m3 block scale, as a packed bf16
// pair. A 2-bit times a 4-bit significand is exact in fp32 and in bf16, so keeping the upper halves
// of the fp32 products converts exactly.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_scaled_to_bf16(uint32_t w, float s) {
  f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  uint32_t a = __builtin_bit_cast(uint32_t, f[0] * s);
  uint32_t b = __builtin_bit_cast(uint32_t, f[1] * s);
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element i % 4 of the 8-byte
// chunks fetched by lanes 4e + i / 4 (e = 0..3). Pointing lane j of a group at row r0 + j / 4,
// columns c0 + 4 (j % 4) .. + 3 of a row-major bf16 tile therefore hands lane i the column c0 + i of
// rows r0 .. r0 + 3: a transposed operand for the MFMA.
__device__ __forceinline__ bf16x4 lds_read_tr16(const char* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float max_across_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

__device__ __forceinline__ float sum_across_groups(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Split fp32 values into NTERM bf16 terms whose sum reproduces them (exactly for NTERM = 3: each term
// carries the next 8+ significant bits of the remainder).
template <int NTERM>
__device__ __forceinline__ void split_terms(const float (&v)[8], bf16x8 (&A)[NTERM]) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = v[e];
#pragma unroll
  for (int k = 0; k < NTERM; ++k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 h = (__bf16)r[e];
      A[k][e] = h;
      r[e] -= (float)h;
    }
  }
}

}  // namespace sda
