// sda_v41.hip -- the V4.1 decode prologue: RoPE on the query dims 448..511 (vLLM swapab_decode_attn,
// stage_inputs: Q RoPE as GPT-J pairs in fp32, rounded to bf16), written to the workspace as [T][H][64];
// the decode kernels read dims 0..447 from q and these 64 from there.
//
// One thread per 16-byte piece (8 dims, four pairs) of the rotated dims of a query row, rotated with the
// cos / sin of pairs 4c .. 4c+3 of the token's position (cos_sin row: cos of pair i at [i], sin at
// [32 + i]; a position outside the table rotates nothing).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_device.h"
#include "sda_internal.h"

namespace sda {

__global__ __launch_bounds__(256) void rope_q_kernel(RopeParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.T * p.H;
  if (i >= rows * 8) return;
  const int64_t row = i >> 3;
  const int c = (int)(i & 7);
  const int t = (int)(row / p.H), h = (int)(row - (int64_t)t * p.H);
  u32x4 x = *(const u32x4*)(p.q + (int64_t)t * p.q_st + (int64_t)h * p.q_sh + 448 + 8 * c);
  {
    const int64_t pos = p.positions[t];
    if (pos >= 0 && pos < p.num_positions) {
      const float* cs = p.cos_sin + pos * p.cs_stride + 4 * c;
      const f32x4 cv = *(const f32x4*)cs;
      const f32x4 sv = *(const f32x4*)(cs + 32);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float qe = __builtin_bit_cast(float, x[k] << 16);
        const float qo = __builtin_bit_cast(float, x[k] & 0xFFFF0000u);
        const float re = __builtin_fmaf(qe, cv[k], -(qo * sv[k]));
        const float ro = __builtin_fmaf(qo, cv[k], qe * sv[k]);
        x[k] = (uint32_t)f32_to_bf16_bits(re) | ((uint32_t)f32_to_bf16_bits(ro) << 16);
      }
    }
  }
  *(u32x4*)(p.q_out + row * 64 + 8 * c) = x;
}

hipError_t launch_rope_q(const RopeParams& p, hipStream_t stream) {
  const int64_t threads = (int64_t)p.T * p.H * 8;
  hipLaunchKernelGGL(rope_q_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sda
