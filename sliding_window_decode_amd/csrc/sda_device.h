// sda_device.h -- gfx950 device helpers shared by the decode-attention kernels: vector types,
// exact fp8/fp4 -> bf16 conversions, LDS transpose reads, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// 16 bytes from an 8-byte aligned address (records of 584 bytes start 8-byte aligned; the load is
// the same global_load_dwordx4 as for a 16-byte aligned one)
typedef const __attribute__((address_space(1))) u32x4 __attribute__((aligned(8))) gbl_u32x4_a8;
__device__ __forceinline__ u32x4 ld_global_16(uint64_t addr) { return *(gbl_u32x4_a8*)addr; }
__device__ __forceinline__ uint32_t ld_global_u16(uint64_t addr) { return *(gbl_u16*)addr; }

// Exact e4m3fn -> bf16 of the 4 codes of a word (the gfx950 conversion decodes the OCP format; every
// e4m3 value has at most 4 significant bits, so the bf16 result is exact).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

// The same with a power-of-two scale applied by the conversion: the scale operand contributes only
// its exponent field, read as an OCP MX E8M0 byte, so passing the float whose exponent field is an ue8m0
// scale byte e multiplies by 2^(e - 127), 2^-127 for e = 0 and NaN for e = 255. Exact while the products
// stay within the bf16 range. Only for the conversions' scale operand: as an fp32 value the same bits are
// 0 for e = 0 and +inf for e = 255 (ue8m0_value gives the value).
__device__ __forceinline__ float ue8m0_scale(uint32_t byte) { return __builtin_bit_cast(float, (byte & 0xFFu) << 23); }

// The value of an ue8m0 scale byte as an fp32 multiplier: 2^(e - 127), with the fp32 denormal 2^-127 for
// e = 0 and NaN for e = 255 (OCP MX E8M0), the values the scaled conversions take from ue8m0_scale.
__device__ __forceinline__ float ue8m0_value(uint32_t byte) {
  const uint32_t b = byte & 0xFFu;
  return __builtin_bit_cast(float, b == 0u ? 0x00400000u : (b == 255u ? 0x7FC00000u : b << 23));
}
__device__ __forceinline__ void e4m3x4_to_bf16_scaled(uint32_t w, float scale, uint32_t& lo, uint32_t& hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, true);
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

// A (token, head)'s output factor and LSE from its running max m and weight sum lt (base 2, the sum over all
// its rows) and the sink logit sink2 (log2 units; -inf without a sink), folded in when the token is whole:
// inv multiplies the accumulated output, lse_out is ln(e^sink + sum e^z) (no rows and no sink: 0 and -inf;
// an infinite sink: 0 and +inf). For a split (whole = false) they normalize the partial, sink left out.
// A NaN sum (a row whose scores are NaN, e.g. an ue8m0 scale byte 255) gives a NaN factor and LSE.
__device__ __forceinline__ void token_output_factor(float m, float lt, float sink2, bool whole, float& inv,
                                                    float& lse_out) {
  // lt * 0 is 0, or NaN for a NaN sum; !(x <= 0) holds for x > 0 and for NaN
  if (whole) {
    const float Mx = fmaxf(m, sink2);
    if (Mx == kNegInf) {
      inv = lt * 0.f;
      lse_out = lt * 0.f + kNegInf;
    } else if (sink2 == kPosInf) {
      inv = 0.f;
      lse_out = kPosInf;
    } else {
      const float fo = (m == kNegInf) ? 0.f : fast_exp2(m - Mx);
      const float den = lt * fo + (sink2 != kNegInf ? fast_exp2(sink2 - Mx) : 0.f);
      const bool pos = !(den <= 0.f);
      inv = pos ? fo / den : 0.f;
      lse_out = pos ? (Mx + __log2f(den)) * kLn2 : kNegInf;
    }
  } else {
    const bool pos = !(lt <= 0.f);
    inv = pos ? 1.0f / lt : 0.f;
    lse_out = pos ? (m + __log2f(lt)) * kLn2 : kNegInf;
  }
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


// ---------------------------------------------------------------- global -> LDS streaming helpers

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void gbl_void;
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Global -> LDS load of 16 (4) bytes per lane: lane l's bytes land at lds_wave_base + 16 l (4 l);
// the base must be the same for the whole wave.
__device__ __forceinline__ void dma16(uint64_t src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)(uintptr_t)src, (lds_void*)lds_wave_base, 16, 0, 0);
}
// f(integral_constant<int, I>) for I = B .. E-1, each I a compile-time constant
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// The same with a constant byte offset OFF in the load's immediate. The hardware adds it to both addresses:
// lane l's 16 bytes come from src + OFF and land at lds_wave_base + OFF + 16 l (probed on gfx950).
template <int OFF>
__device__ __forceinline__ void dma16_at(uint64_t src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)(uintptr_t)src, (lds_void*)lds_wave_base, 16, OFF, 0);
}
__device__ __forceinline__ void dma4(uint64_t src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)(uintptr_t)src, (lds_void*)lds_wave_base, 4, 0, 0);
}

// Workgroup barrier that does not wait for the gathers in flight (only for this wave's LDS
// operations). The compiler's __syncthreads would also drain every global -> LDS load.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ds_read_b64_tr_b8 (see lds_read_tr16 for the lane pattern; here 8 one-byte elements from lanes
// 2e + i / 8). Issued as inline assembly: with the builtin the compiler drains every global -> LDS
// load in flight before the read, as it cannot tell that the two touch different ring buffers. The
// result may only be used after an explicit s_waitcnt lgkmcnt that names it as an operand.
__device__ __forceinline__ i32x2 lds_tr8(uint32_t lds_addr) {
  i32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}

// An 8-byte LDS read that waits for itself (and every LDS operation before it) in the same statement, so
// that the compiler can neither hoist it nor hold its result across the code around it.
__device__ __forceinline__ uint64_t lds_read_u64_waited(uint32_t lds_addr) {
  uint64_t r;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(lds_addr) : "memory");
  return r;
}

// ds_read_b64_tr_b16 as inline assembly, for the same reason as lds_tr8 and under the same rule.
__device__ __forceinline__ i32x2 lds_tr16(uint32_t lds_addr) {
  i32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 e4m3 codes times 2^(e - 127) -> two bf16x8 (the scaled conversion above).
__device__ __forceinline__ void e4m3x16_to_bf16_scaled(const u32x4 x, float scale, bf16x8& lo, bf16x8& hi) {
  uint32_t y[8];
  e4m3x4_to_bf16_scaled(x[0], scale, y[0], y[1]);
  e4m3x4_to_bf16_scaled(x[1], scale, y[2], y[3]);
  e4m3x4_to_bf16_scaled(x[2], scale, y[4], y[5]);
  e4m3x4_to_bf16_scaled(x[3], scale, y[6], y[7]);
  lo = __builtin_bit_cast(bf16x8, u32x4{y[0], y[1], y[2], y[3]});
  hi = __builtin_bit_cast(bf16x8, u32x4{y[4], y[5], y[6], y[7]});
}

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(const i32x2 x) {
  uint32_t y[4];
  e4m3x4_to_bf16((uint32_t)x[0], y[0], y[1]);
  e4m3x4_to_bf16((uint32_t)x[1], y[2], y[3]);
  return __builtin_bit_cast(bf16x8, u32x4{y[0], y[1], y[2], y[3]});
}

// s_waitcnt vmcnt(N): at most N global operations of this wave still pending (they complete in issue
// order).
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int LO, int HI>
__device__ __forceinline__ void vm_wait_tree(int n) {
  if constexpr (LO == HI) {
    vm_wait<LO>();
  } else {
    constexpr int MID = (LO + HI + 1) / 2;
    if (n >= MID)
      vm_wait_tree<MID, HI>(n);
    else
      vm_wait_tree<LO, MID - 1>(n);
  }
}

// Waits until at most n global operations of this wave are pending (n is wave-uniform): exactly n up
// to 31, and 32 for larger n (then more is waited for than needed, never less).
__device__ __forceinline__ void vm_wait_atmost(int n) {
  if (n >= 32)
    vm_wait<32>();
  else
    vm_wait_tree<0, 31>(n);
}

}  // namespace sda
