// sda_sched.hip -- the split scheduler and the LSE combine kernel.
//
// Scheduler (FlashMLA sparse_decode.h: get_decoding_sched_meta, DecodeImplMeta): every token costs
// max(1, ceil(n_main/64) + ceil(n_extra/64)) tiles plus a fixed overhead F; the concatenated
// (token, tile) sequence is cut into num_parts contiguous parts of equal cost (see sda_internal.h).
// Combine (FlashMLA run_flash_mla_combine_kernel; vLLM swapab_decode_attn step 9): LSE-weighted sum
// of the normalized partials of every split token, the sink folded into the denominator once. In a
// V4.1 call every token comes through here and leaves as MXFP8 (vLLM swapab_decode_attn step 9: the
// inverse RoPE of dims 448..511 and the cast with one ue8m0 scale per 32 dims).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_device.h"
#include "sda_internal.h"

namespace sda {

// Inclusive prefix sum over the block (wave shuffles, one barrier for the wave totals).
__device__ int block_incl_scan(int v, int* wave_tot, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) wave_tot[wave] = v;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = wave_tot[w];
    before += (w < wave) ? x : 0;
    all += x;
  }
  __syncthreads();
  total = all;
  return v + before;
}

__global__ __launch_bounds__(1024) void sched_kernel(SchedParams p) {
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x;
  const int NT = blockDim.x;
  // the first chunk's token (every token when T <= NT, the launch's usual shape): lengths read once,
  // and its cost scan gives the total too
  int n0c = 0, n1c = 0, costc = 0;
  if (tid < p.T) {
    n0c = clamp_len(p.lens[0], p.lens_div[0], p.width[0], tid);
    n1c = p.nlists > 1 ? clamp_len(p.lens[1], p.lens_div[1], p.width[1], tid) : 0;
    costc = token_tiles(n0c, n1c) + p.F;
  }
  int local = costc;
  for (int t = tid + NT; t < p.T; t += NT) {
    const int n0 = clamp_len(p.lens[0], p.lens_div[0], p.width[0], t);
    const int n1 = p.nlists > 1 ? clamp_len(p.lens[1], p.lens_div[1], p.width[1], t) : 0;
    local += token_tiles(n0, n1) + p.F;
  }
  int total = 0;
  const int incl0 = block_incl_scan(local, wave_tot, total);
  const int Q = (int)part_quantum(total, p.num_parts);
  const bool one_chunk = p.T <= NT;
  int carry = 0, split_carry = 0;
  for (int base = 0; base < p.T; base += NT) {
    const int t = base + tid;
    int nt = 0, cost = 0, n0 = 0, n1 = 0, cum = 0, chunk_cost = 0;
    if (one_chunk) {  // base == 0: the scan above is this chunk's
      n0 = n0c;
      n1 = n1c;
      cost = costc;
      nt = t < p.T ? cost - p.F : 0;
      cum = incl0 - cost;
      chunk_cost = total;
    } else {
      if (t < p.T) {
        n0 = clamp_len(p.lens[0], p.lens_div[0], p.width[0], t);
        n1 = p.nlists > 1 ? clamp_len(p.lens[1], p.lens_div[1], p.width[1], t) : 0;
        nt = token_tiles(n0, n1);
        cost = nt + p.F;
      }
      cum = carry + block_incl_scan(cost, wave_tot, chunk_cost) - cost;  // cost-axis start of t
    }
    int nsplit = 0, pos0 = 0, p0 = 0, p1 = 0;
    if (t < p.T) {
      pos0 = cum + p.F;  // position of the token's first tile
      p0 = pos0 / Q;
      p1 = (pos0 + nt - 1) / Q;
      nsplit = p1 - p0 + 1;
    }
    int chunk_splits = 0;
    const int sincl = block_incl_scan(nsplit, wave_tot, chunk_splits);
    if (t < p.T) {
      const int s_first = split_carry + sincl - nsplit;
      p.num_splits[t] = s_first;
      const int prev_last = (cum == 0) ? -1 : (cum - 1) / Q;  // part of the previous token's last tile
      for (int pp = prev_last + 1; pp <= p1; ++pp) {
        const int bi = pp * Q - pos0 > 0 ? pp * Q - pos0 : 0;
        int32_t* m = p.meta + (int64_t)pp * SDA_META_INTS;
        m[0] = t;
        m[1] = bi;
        m[4] = (pp >= p0) ? pp - p0 : 0;
        m[5] = n0;
        m[6] = n1;
        m[7] = s_first;
        if (pp > 0) {
          int32_t* mp = p.meta + (int64_t)(pp - 1) * SDA_META_INTS;
          mp[2] = t;
          mp[3] = bi;
        }
      }
    }
    carry += chunk_cost;
    split_carry += chunk_splits;
  }
  const int last = (total - 1) / Q;  // part of the very last tile
  for (int pp = last + 1 + tid; pp < p.num_parts; pp += NT) {
    int32_t* m = p.meta + (int64_t)pp * SDA_META_INTS;
    m[0] = p.T; m[1] = 0; m[2] = p.T; m[3] = 0; m[4] = 0; m[5] = 0; m[6] = 0; m[7] = 0;
  }
  if (tid == 0) {
    int32_t* m = p.meta + (int64_t)last * SDA_META_INTS;
    m[2] = p.T;
    m[3] = 0;
    p.num_splits[p.T] = split_carry;
  }
}

// One workgroup per (token, block of 16 heads), one wave per head: lane l owns dims 8l .. 8l+7, so every
// load and store of a row is contiguous across the wave. The splits are read four at a time with every
// load of a batch issued before any is used (a token rarely has more than a few splits), so a merge
// costs about one global round trip per batch.
//
// V4.1 instance: every token comes through, and each (head, 32-dim chunk) leaves as MXFP8 (vLLM
// swapab_decode_attn step 9): x = the merged output (0 when the token has no rows or an infinite sink),
// its dims 448..511 rotated back per GPT-J pair in fp32, then amax over the chunk (four lanes) =
// max(max |x|, 1e-10), scale byte = ue8m0 of amax * (1/448) rounded up to a power of two, codes =
// e4m3(x * 2^(127 - byte)) (v_cvt_pk_fp8_f32: round to nearest even; |x * 2^(127 - byte)| stays within
// 448 up to one rounding of the product, which still rounds to 448).
template <bool V41>
__global__ __launch_bounds__(1024) void combine_kernel(CombineParams p) {
  const int t = blockIdx.x;
  // no num_splits array (a whole-token call): token t is its own single split, number t
  const int s0 = p.num_splits ? p.num_splits[t] : t;
  const int n = p.num_splits ? p.num_splits[t + 1] - s0 : 1;
  if (n < (V41 ? 1 : 2)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = blockIdx.y * 16 + (tid >> 6);
  const int d0 = 8 * lane;
  const bool has_sink = p.sink != nullptr;
  const float sk = has_sink ? p.sink[h] : kNegInf;
  // V4.1: the cos / sin of the lane's four pairs, loaded before the merge so that their latency overlaps
  // that of the partials (identity for a position outside the table)
  f32x4 rc = f32x4{1.f, 1.f, 1.f, 1.f}, rs = f32x4{0.f, 0.f, 0.f, 0.f};
  bool rot = false;
  if constexpr (V41) {
    if (d0 >= 448) {
      const int64_t pos = p.positions[t];
      if (pos >= 0 && pos < p.num_positions) {
        const float* cs = p.cos_sin + pos * p.cs_stride + (d0 - 448) / 2;  // pairs (d0 - 448) / 2 .. + 3
        rc = *(const f32x4*)cs;
        rs = *(const f32x4*)(cs + 32);
        rot = true;
      }
    }
  }
  constexpr int KB = 4;  // splits per batch
  // running merge state: max M, denominator den and accumulator relative to M
  float M = sk;
  float den = has_sink ? 1.0f : 0.0f;  // exp(sk - M) with M = sk
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  bool nan_part = false;  // a partial with a NaN LSE (a NaN in its rows) makes the token NaN
  for (int k0 = 0; k0 < n; k0 += KB) {
    float lk[KB];
    f32x4 v[KB][2];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int k = k0 + j < n ? k0 + j : k0;  // a duplicate read beyond the end, weighted 0 below
      lk[j] = p.lse_acc[(int64_t)(s0 + k) * p.H + h];
      const f32x4* src = (const f32x4*)(p.o_acc + ((int64_t)(s0 + k) * p.H + h) * kDv + d0);
      v[j][0] = src[0];
      v[j][1] = src[1];
    }
    float bm = M;
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (k0 + j < n) {
        bm = fmaxf(bm, lk[j]);
        nan_part |= lk[j] != lk[j];
      }
    if (bm == kNegInf || bm == kPosInf) {
      M = bm;
      continue;
    }
    const float r = (M == kNegInf) ? 0.f : expf(M - bm);  // rescale what was merged so far
    den *= r;
    acc[0] *= r;
    acc[1] *= r;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const float wj = (k0 + j < n && lk[j] != kNegInf) ? expf(lk[j] - bm) : 0.f;
      den += wj;
      acc[0] += wj * v[j][0];
      acc[1] += wj * v[j][1];
    }
    M = bm;
  }
  if (nan_part) {
    M = __builtin_nanf("");
    den = M;
  }
  const bool ok = !(M == kNegInf || M == kPosInf);
  if constexpr (V41) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = ok ? acc[0][k] / den : 0.f;
      x[4 + k] = ok ? acc[1][k] / den : 0.f;
    }
    if (rot) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float oe = x[2 * j], oo = x[2 * j + 1];
        x[2 * j] = __builtin_fmaf(oe, rc[j], rs[j] * oo);
        x[2 * j + 1] = __builtin_fmaf(oo, rc[j], -(rs[j] * oe));
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));  // the chunk's four lanes
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, 1e-10f);
    const uint32_t yb = __builtin_bit_cast(uint32_t, amax * (float)(1.0 / 448.0));
    const uint32_t ex = ((yb >> 23) & 0xFFu) + ((yb & 0x7FFFFFu) != 0u ? 1u : 0u);
    const float inv = __builtin_bit_cast(float, (254u - ex) << 23);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[1] * inv, 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * inv, x[3] * inv, w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] * inv, x[5] * inv, 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] * inv, x[7] * inv, w1, true);
    *(u32x2*)(p.o8 + (int64_t)t * p.o8_st + (int64_t)h * p.o8_sh + d0) = u32x2{(uint32_t)w0, (uint32_t)w1};
    if ((lane & 3) == 0) p.osc[(int64_t)t * p.osc_st + (int64_t)h * p.osc_sh + (lane >> 2)] = (uint8_t)ex;
    if (p.lse && lane == 0) p.lse[(int64_t)t * p.l_st + h] = ok ? M + logf(den) : M;
    return;
  }
  uint16_t* orow = p.out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + d0;
  if (!ok) {
    *(u32x4*)orow = u32x4{0u, 0u, 0u, 0u};
    if (lane == 0) p.lse[(int64_t)t * p.l_st + h] = M;
    return;
  }
  const float inv = 1.0f / den;
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4& a = acc[q >> 1];
    const int k = (q & 1) * 2;
    o[q] = (uint32_t)f32_to_bf16_bits(a[k] * inv) | ((uint32_t)f32_to_bf16_bits(a[k + 1] * inv) << 16);
  }
  *(u32x4*)orow = o;
  if (lane == 0) p.lse[(int64_t)t * p.l_st + h] = M + logf(den);
}

hipError_t launch_sched(const SchedParams& p, hipStream_t stream) {
  const int threads = p.T >= 1024 ? 1024 : ((p.T + 63) / 64) * 64;
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  if (p.o8)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(p.T, p.H / 16), dim3(1024), 0, stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(p.T, p.H / 16), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sda
