// sda_kernels.hip -- gfx950 kernels of the decode-attention library: the split scheduler, the
// split-KV decode kernel and the LSE combine.
//
// Decode kernel outline (one workgroup = one scheduler part x one group of query heads):
//   for every token the part touches:
//     Q of the wave's 16 heads -> registers (bf16 MFMA B operand layout)
//     for every 64-position tile of the token inside the part:
//       gather: slot ids -> record addresses (masking -1 / out-of-range / past-length positions),
//               coalesced 16-byte loads of the records, exact dequant of the codes to bf16 into a
//               row-major LDS tile; fp32 scales go to a small LDS table
//       S^T[rows x heads] = K . Q^T with v_mfma_f32_16x16x32_bf16 (rows on M: the score layout
//               is then directly the A operand of the PV product); scales applied to the fp32
//               scores (per slot, or per 128-dim group with one accumulator per group)
//       online softmax in base 2 (max and sums across the wave with lane shuffles)
//       O[heads x 512] += P' . V with v_mfma_f32_16x16x32_bf16, V read transposed from the same
//               LDS tile with ds_read_b64_tr_b16; P' = p * scale split into `NTERM` bf16 terms
//     merge the waves that processed different row slices, then either the final bf16 output and
//     LSE (with the sink) or a normalized fp32 partial for the combine kernel.
// Sources: masked softmax attention (native_swa_decode.py, _fallback_batched_sdp); gather,
// validity and page addressing (vLLM swapab_decode_attn, stage_inputs); online softmax with a
// running max (native_swa_decode.py, BlackwellSWADecodeKernel); sink and LSE merge (vLLM
// swapab_decode_attn, device kernel step 9); scheduler and split buffers (FlashMLA
// sparse_decode.h, get_decoding_sched_meta call and o_accum/lse_accum).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_internal.h"

namespace sda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kPosInf = __builtin_inff();

// ---------------------------------------------------------------- small helpers

// 16-byte chunk c of LDS row r is stored at chunk position (c & ~7) | ((c ^ f(r)) & 7),
// f(r) = 2 (r % 4) + (r / 4) % 2: eight consecutive rows at one chunk and four consecutive rows at
// two adjacent chunks both land on distinct 16-byte bank groups of a 128-byte window.
__device__ __forceinline__ int swz(int c, int r) {
  int f = ((r & 3) << 1) | ((r >> 2) & 1);
  return (c & ~7) | ((c ^ f) & 7);
}

__device__ __forceinline__ float wave_max_across_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum_across_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exact e4m3fn -> bf16 of the 4 codes of a word (hardware conversion, OCP format on gfx950).
__device__ __forceinline__ void e4m3x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(byte, false)[0];
}

// Two e2m1 codes of byte `sel` of w, times an e4m3 block scale, as a packed bf16 pair. The product
// of a 2-bit and a 4-bit significand is exact in fp32 and in bf16, so taking the upper halves of
// the fp32 words is an exact conversion.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_scaled_to_bf16(uint32_t w, float s) {
  f32x2 f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  uint32_t a = __builtin_bit_cast(uint32_t, f[0] * s);
  uint32_t b = __builtin_bit_cast(uint32_t, f[1] * s);
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef const __attribute__((address_space(1))) u32x4 gbl_u32x4;
typedef const __attribute__((address_space(1))) uint16_t gbl_u16;

__device__ __forceinline__ u32x4 ld_global_16(uint64_t addr) { return *(gbl_u32x4*)addr; }
__device__ __forceinline__ uint32_t ld_global_u16(uint64_t addr) { return *(gbl_u16*)addr; }

__device__ __forceinline__ bf16x4 lds_read_tr16(const char* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// ---------------------------------------------------------------- scheduler

// Inclusive block-wide prefix sum (Hillis-Steele); `total` receives the sum over the block.
template <typename TV>
__device__ TV block_incl_scan(TV v, TV* sh, TV& total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const TV add = (tid >= off) ? sh[tid - off] : (TV)0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const TV r = sh[tid];
  total = sh[blockDim.x - 1];
  __syncthreads();
  return r;
}

// One workgroup. Pass 1 sums the token costs; pass 2 rescans them chunk by chunk and writes, for
// every token, its split count prefix and the begin/end records of the parts that start in it.
__global__ __launch_bounds__(1024) void sched_kernel(SchedParams p) {
  __shared__ int64_t s64[1024];
  __shared__ int32_t s32[1024];
  const int tid = threadIdx.x;
  const int NT = blockDim.x;
  int64_t local = 0;
  for (int t = tid; t < p.T; t += NT) {
    const int n0 = clamp_len(p.lens[0], p.width[0], t);
    const int n1 = p.nlists > 1 ? clamp_len(p.lens[1], p.width[1], t) : 0;
    local += token_tiles(n0, n1) + p.F;
  }
  int64_t total = 0;
  (void)block_incl_scan<int64_t>(local, s64, total);
  const int64_t Q = part_quantum(total, p.num_parts);
  int64_t carry = 0;
  int32_t split_carry = 0;
  for (int base = 0; base < p.T; base += NT) {
    const int t = base + tid;
    int nt = 0;
    int64_t cost = 0;
    if (t < p.T) {
      const int n0 = clamp_len(p.lens[0], p.width[0], t);
      const int n1 = p.nlists > 1 ? clamp_len(p.lens[1], p.width[1], t) : 0;
      nt = token_tiles(n0, n1);
      cost = nt + p.F;
    }
    int64_t chunk_cost = 0;
    const int64_t incl = block_incl_scan<int64_t>(cost, s64, chunk_cost);
    const int64_t cum = carry + incl - cost;  // cost-axis start of token t
    int32_t nsplit = 0;
    int64_t pos0 = 0, p0 = 0, p1 = 0;
    if (t < p.T) {
      pos0 = cum + p.F;                       // position of the token's first tile
      p0 = pos0 / Q;
      p1 = (pos0 + nt - 1) / Q;
      nsplit = (int32_t)(p1 - p0 + 1);
    }
    int32_t chunk_splits = 0;
    const int32_t sincl = block_incl_scan<int32_t>(nsplit, s32, chunk_splits);
    if (t < p.T) {
      p.num_splits[t] = split_carry + sincl - nsplit;
      const int64_t prev_last = (cum == 0) ? -1 : (cum - 1) / Q;  // part of the previous token's last tile
      for (int64_t pp = prev_last + 1; pp <= p1; ++pp) {
        int64_t bi = pp * Q - pos0;
        if (bi < 0) bi = 0;
        int32_t* m = p.meta + pp * SDA_META_INTS;
        m[0] = t;
        m[1] = (int32_t)bi;
        m[4] = (pp >= p0) ? (int32_t)(pp - p0) : 0;
        m[5] = 0;
        m[6] = 0;
        m[7] = 0;
        if (pp > 0) {
          int32_t* mp = p.meta + (pp - 1) * SDA_META_INTS;
          mp[2] = t;
          mp[3] = (int32_t)bi;
        }
      }
    }
    carry += chunk_cost;
    split_carry += chunk_splits;
  }
  const int64_t last = (total - 1) / Q;  // part of the very last tile
  for (int64_t pp = last + 1 + tid; pp < p.num_parts; pp += NT) {
    int32_t* m = p.meta + pp * SDA_META_INTS;
    m[0] = p.T; m[1] = 0; m[2] = p.T; m[3] = 0; m[4] = 0; m[5] = 0; m[6] = 0; m[7] = 0;
  }
  if (tid == 0) {
    int32_t* m = p.meta + last * SDA_META_INTS;
    m[2] = p.T;
    m[3] = 0;
    p.num_splits[p.T] = split_carry;
  }
}

// ---------------------------------------------------------------- decode kernel

template <int DQK>
struct TileSmem {
  static constexpr int RS = DQK * 2;  // bytes per LDS row (bf16)
  char tile[kTileRows * RS];
  uint64_t addr[kTileRows];
  float scale[kTileRows][4];
  int valid[kTileRows];
  int any_valid;
};

// Gather one tile: 64 list positions [pos0, pos0 + 64) of list `ld` for token t (n = clamped length).
template <int DQK, int NT>
__device__ __forceinline__ void gather_tile(TileSmem<DQK>& sm, const ListDev& ld, int t, int pos0, int n) {
  constexpr int RS = TileSmem<DQK>::RS;
  const int tid = threadIdx.x;
  if (tid == 0) sm.any_valid = 0;
  __syncthreads();
  if (tid < kTileRows) {
    const int pos = pos0 + tid;
    int sid = -1;
    if (pos < n) sid = ld.idx[(int64_t)t * ld.row_stride + pos];
    const bool ok = sid >= 0 && sid < ld.slots;
    uint64_t a = 0;
    if (ok) {
      const uint32_t pg = (uint32_t)sid >> ld.page_shift;
      const uint32_t off = (uint32_t)sid & ((1u << ld.page_shift) - 1u);
      a = (uint64_t)ld.base + (uint64_t)pg * (uint64_t)ld.page_stride + (uint64_t)off * (uint64_t)ld.rec;
    }
    sm.addr[tid] = a;
    sm.valid[tid] = ok ? 1 : 0;
    if (ld.format == SDA_FP8_SLOTSCALE || ld.format == SDA_NVFP4_288) {
      // one scale for the whole row: the slot's fp32 scale, or 1 (NVFP4 block scales are applied
      // exactly during the conversion to bf16)
      const float s = ok ? (ld.format == SDA_FP8_SLOTSCALE ? ld.slot_scale[sid] : 1.0f) : 0.0f;
      sm.scale[tid][0] = s;
      sm.scale[tid][1] = s;
      sm.scale[tid][2] = s;
      sm.scale[tid][3] = s;
    }
    if (ok) sm.any_valid = 1;
  }
  __syncthreads();
  if (!sm.any_valid) return;
  if (ld.format == SDA_NVFP4_288) {
    // 16 packed chunks per row; chunk c = dims [32c, 32c + 32), scales = bytes 2c, 2c+1 of the scale block
    for (int u = tid; u < kTileRows * 16; u += NT) {
      const int r = u >> 4, c = u & 15;
      const uint64_t a = sm.addr[r];
      u32x4 v = {0u, 0u, 0u, 0u};
      uint32_t sb = 0;
      if (a) {
        v = ld_global_16(a + 16 * c);
        sb = ld_global_u16(a + 256 + 2 * c);
      }
      const float s0 = e4m3_to_f32(sb & 0xFFu), s1 = e4m3_to_f32(sb >> 8);
      char* row = sm.tile + r * RS;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s = q < 2 ? s0 : s1;
        u32x4 o;
        o[0] = e2m1x2_scaled_to_bf16<0>(v[q], s);
        o[1] = e2m1x2_scaled_to_bf16<1>(v[q], s);
        o[2] = e2m1x2_scaled_to_bf16<2>(v[q], s);
        o[3] = e2m1x2_scaled_to_bf16<3>(v[q], s);
        *(u32x4*)(row + 16 * swz(4 * c + q, r)) = o;
      }
    }
  } else {
    // 32 chunks of 16 e4m3 codes per row: chunk c = dims [16c, 16c + 16)
    for (int u = tid; u < kTileRows * 32; u += NT) {
      const int r = u >> 5, c = u & 31;
      const uint64_t a = sm.addr[r];
      u32x4 v = {0u, 0u, 0u, 0u};
      if (a) v = ld_global_16(a + 16 * c);
      uint32_t w[8];
      e4m3x4_to_bf16(v[0], w[0], w[1]);
      e4m3x4_to_bf16(v[1], w[2], w[3]);
      e4m3x4_to_bf16(v[2], w[4], w[5]);
      e4m3x4_to_bf16(v[3], w[6], w[7]);
      const u32x4 o0 = {w[0], w[1], w[2], w[3]};
      const u32x4 o1 = {w[4], w[5], w[6], w[7]};
      char* row = sm.tile + r * RS;
      *(u32x4*)(row + 16 * swz(2 * c, r)) = o0;
      *(u32x4*)(row + 16 * swz(2 * c + 1, r)) = o1;
    }
    if (ld.format != SDA_FP8_SLOTSCALE) {
      for (int r = tid; r < kTileRows; r += NT) {
        const uint64_t a = sm.addr[r];
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if (a) s = __builtin_bit_cast(f32x4, ld_global_16(a + 512));
        sm.scale[r][0] = s[0];
        sm.scale[r][1] = s[1];
        sm.scale[r][2] = s[2];
        sm.scale[r][3] = s[3];
      }
    }
    if constexpr (DQK == 576) {
      // 64 bf16 rope dims at bytes [528, 656): LDS chunks 64..71
      for (int u = tid; u < kTileRows * 8; u += NT) {
        const int r = u >> 3, c = u & 7;
        const uint64_t a = sm.addr[r];
        u32x4 v = {0u, 0u, 0u, 0u};
        if (a) v = ld_global_16(a + 528 + 16 * c);
        *(u32x4*)(sm.tile + r * RS + 16 * swz(64 + c, r)) = v;
      }
    }
  }
  __syncthreads();
}

// Split fp32 values into NTERM bf16 terms whose sum reproduces them (exactly for NTERM = 3).
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

// One tile of one wave: S^T = K Q^T, online softmax update, O += P' V.
// Every row carries four fp32 scales, one per 128 dims of the e4m3 codes (a per-slot scale is stored
// four times, NVFP4 rows carry 1); `row_scaled` says the four are equal, so P' is split only once.
//
// LDS addressing: rows handled by a wave start at multiples of 8, so the swizzle term f(row) of a lane
// is the same for every row it touches; `lb` holds the per-lane base addresses and every access is
// base + a compile-time offset.
struct LaneBases {
  const char* k[2];  // K operand: chunk parity 0 / 1
  const char* v[4];  // V operand (transposed read): chunk pair index db % 4
};

template <int DQK, int NRS>
__device__ __forceinline__ LaneBases lane_bases(const TileSmem<DQK>& sm, int rs) {
  constexpr int RS = TileSmem<DQK>::RS;
  constexpr int RPW = kTileRows / NRS;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const int row0 = rs * RPW;
  LaneBases b;
  {
    const int ra = row0 + li;
    const int f = ((ra & 3) << 1) | ((ra >> 2) & 1);
    const int xe = G ^ f;  // chunk 4 ks + G, even ks
    b.k[0] = sm.tile + ra * RS + 16 * xe;
    b.k[1] = sm.tile + ra * RS + 16 * (xe ^ 4);
  }
  {
    const int rv = row0 + 4 * G + (li >> 2);
    const int f = ((rv & 3) << 1) | ((rv >> 2) & 1);
    const int cb = (li & 3) >> 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) b.v[q] = sm.tile + rv * RS + 16 * ((2 * q + cb) ^ f) + 8 * (li & 1);
  }
  return b;
}

template <int DQK, int NRS, int NTERM>
__device__ __forceinline__ void compute_tile(const TileSmem<DQK>& sm, const LaneBases& lb,
                                             const bf16x8 (&qreg)[DQK / 32], f32x4 (&O)[32], float& m, float& l,
                                             int rs, float scale_log2, bool row_scaled) {
  constexpr int RS = TileSmem<DQK>::RS;
  constexpr int RPW = kTileRows / NRS;
  constexpr int NRB = RPW / 16;
  constexpr int NKS = DQK / 32;
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4, li = lane & 15;
  const int row0 = rs * RPW;

  // ---- QK^T (swap-AB: rows on M, heads on N); one partial per 128-dim scale group
  f32x4 S[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ks = 4 * g + kk;
        const bf16x8 a = *(const bf16x8*)(lb.k[ks & 1] + rb * 16 * RS + 128 * (ks >> 1));
        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], part, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += part[r] * sm.scale[row0 + rb * 16 + 4 * G + r][g];
    }
#pragma unroll
    for (int ks = 16; ks < NKS; ++ks) {  // bf16 dims 512..575 carry no scale
      const bf16x8 a = *(const bf16x8*)(lb.k[ks & 1] + rb * 16 * RS + 128 * (ks >> 1));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], acc, 0, 0, 0);
    }
    S[rb] = acc;
    __builtin_amdgcn_sched_barrier(0);  // keep one row block's loads in flight at a time
  }

  // ---- online softmax (base 2). Lane (head li, G) holds rows 16 rb + 4 G + r.
  float tmax = kNegInf;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + rb * 16 + 4 * G + r;
      const float z = sm.valid[row] ? S[rb][r] * scale_log2 : kNegInf;
      S[rb][r] = z;
      tmax = fmaxf(tmax, z);
    }
  }
  tmax = wave_max_across_groups(tmax);
  // The reference max only moves when the tile max exceeds it by more than 8 (log2 units): weights
  // stay <= 2^8, exact in fp32 and in the bf16 term split, and O is rescaled rarely.
  const bool bump = tmax > m + 8.0f;
  const float m_new = bump ? tmax : m;
  const float alpha = bump ? fast_exp2(m - m_new) : 1.0f;  // m = -inf -> 0
  float psum = 0.f;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pz = (m_new == kNegInf) ? 0.0f : fast_exp2(S[rb][r] - m_new);
      S[rb][r] = pz;
      psum += pz;
    }
  }
  l = l * alpha + psum;
  m = m_new;
  if (__any(bump)) {
    float ar[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * G + r);
#pragma unroll
    for (int db = 0; db < 32; ++db) {
#pragma unroll
      for (int r = 0; r < 4; ++r) O[db][r] *= ar[r];
      if (db % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- O += P' V: P' = p * scale (of the output dims' group); V read transposed from the
  // row-major tile with ds_read_b64_tr_b16 (lane i of a 16-lane group receives 4 consecutive rows of
  // column i: exactly the B operand layout, k = the rows in the order of the score layout)
#pragma unroll
  for (int ks = 0; ks < RPW / 32; ++ks) {
    float pv[8];
    int rows[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pv[e] = S[2 * ks][e];
      pv[4 + e] = S[2 * ks + 1][e];
      rows[e] = row0 + 32 * ks + 4 * G + e;
      rows[4 + e] = row0 + 32 * ks + 16 + 4 * G + e;
    }
    bf16x8 A[NTERM];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g == 0 || !row_scaled) {
        float pg[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pg[e] = pv[e] * sm.scale[rows[e]][g];
        split_terms<NTERM>(pg, A);
      }
#pragma unroll
      for (int d8 = 0; d8 < 8; ++d8) {
        const int db = 8 * g + d8;
        const char* vb = lb.v[db & 3] + 32 * ks * RS + 128 * (db >> 2);
        const bf16x4 v0 = lds_read_tr16(vb);
        const bf16x4 v1 = lds_read_tr16(vb + 16 * RS);
        const bf16x8 B = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int k = 0; k < NTERM; ++k) O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[k], B, O[db], 0, 0, 0);
        if (d8 % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

template <int NHB, int NRS, int DQK, int NTERM>
__global__ __launch_bounds__(NHB * NRS * 64) void decode_kernel(DecodeParams p) {
  constexpr int NW = NHB * NRS;
  constexpr int NT = NW * 64;
  constexpr int NKS = DQK / 32;
  static_assert(NRS == 1 || NRS == 2, "row slices");
  static_assert(kTileRows / NRS >= 32, "a wave needs at least 32 rows per tile");
  __shared__ TileSmem<DQK> sm;
  __shared__ float s_stat[NHB][NRS][2][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hb = wave % NHB, rs = wave / NHB;
  const int G = lane >> 4, li = lane & 15;
  const int h0 = blockIdx.y * (16 * NHB) + hb * 16;

  const int32_t* mt = p.meta + (int64_t)blockIdx.x * SDA_META_INTS;
  const int bt = mt[0], bi = mt[1], et = mt[2], ei = mt[3], bk = mt[4];
  if (bt > et || (bt == et && bi >= ei) || bt >= p.T) return;
  const int t_last = (ei > 0) ? et : et - 1;

  for (int t = bt; t <= t_last && t < p.T; ++t) {
    const int n0 = clamp_len(p.lst[0].lens, p.lst[0].width, t);
    const int n1 = p.nlists > 1 ? clamp_len(p.lst[1].lens, p.lst[1].width, t) : 0;
    const int tm = (n0 + kTileRows - 1) / kTileRows;
    const int nt = token_tiles(n0, n1);
    const int i_begin = (t == bt) ? bi : 0;
    const int i_end = (t == et) ? ei : nt;
    const int split_k = (t == bt) ? bk : 0;
    const int s_first = p.num_splits[t];
    const int nsplit = p.num_splits[t + 1] - s_first;

    bf16x8 qreg[NKS];
    {
      const uint16_t* qp = p.q + (int64_t)t * p.q_st + (int64_t)(h0 + li) * p.q_sh + 8 * G;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qreg[ks] = *(const bf16x8*)(qp + 32 * ks);
    }
    f32x4 O[32];
#pragma unroll
    for (int db = 0; db < 32; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    const LaneBases lb = lane_bases<DQK, NRS>(sm, rs);
    float m = kNegInf, l = 0.f;

    for (int i = i_begin; i < i_end; ++i) {
      const int L = (i < tm) ? 0 : 1;
      const int pos0 = kTileRows * (L == 0 ? i : i - tm);
      const int n = (L == 0) ? n0 : n1;
      const ListDev& ld = p.lst[L];
      __syncthreads();  // the previous tile (or merge area) is no longer read
      gather_tile<DQK, NT>(sm, ld, t, pos0, n);
      if (!sm.any_valid) continue;
      const bool row_scaled = ld.format == SDA_FP8_SLOTSCALE || ld.format == SDA_NVFP4_288;
      compute_tile<DQK, NRS, NTERM>(sm, lb, qreg, O, m, l, rs, p.scale_log2, row_scaled);
    }
    l = wave_sum_across_groups(l);

    // ---- merge the row slices of each head block (wave rs = 0 keeps the result)
    if constexpr (NRS > 1) {
      __syncthreads();
      float* xo = (float*)sm.tile;  // [NHB][NRS-1][32][64][4]
      if (rs > 0) {
        float* dst = xo + ((hb * (NRS - 1) + (rs - 1)) * 32 * 64) * 4;
#pragma unroll
        for (int db = 0; db < 32; ++db) *(f32x4*)(dst + (db * 64 + lane) * 4) = O[db];
        if (G == 0) {
          s_stat[hb][rs][0][li] = m;
          s_stat[hb][rs][1][li] = l;
        }
      }
      __syncthreads();
      if (rs > 0) continue;
      float M = m;
#pragma unroll
      for (int r2 = 1; r2 < NRS; ++r2) M = fmaxf(M, s_stat[hb][r2][0][li]);
      const float fs = (m == kNegInf) ? 0.f : fast_exp2(m - M);
      float Lsum = l * fs;
      float fr[NRS];
#pragma unroll
      for (int r2 = 1; r2 < NRS; ++r2) {
        const float mr = s_stat[hb][r2][0][li];
        fr[r2] = (mr == kNegInf) ? 0.f : fast_exp2(mr - M);
        Lsum += s_stat[hb][r2][1][li] * fr[r2];
      }
      float fsr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) fsr[r] = __shfl(fs, 4 * G + r);
#pragma unroll
      for (int db = 0; db < 32; ++db) {
#pragma unroll
        for (int r = 0; r < 4; ++r) O[db][r] *= fsr[r];
      }
#pragma unroll
      for (int r2 = 1; r2 < NRS; ++r2) {
        float frr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) frr[r] = __shfl(fr[r2], 4 * G + r);
        const float* src = xo + ((hb * (NRS - 1) + (r2 - 1)) * 32 * 64) * 4;
#pragma unroll
        for (int db = 0; db < 32; ++db) {
          const f32x4 v = *(const f32x4*)(src + (db * 64 + lane) * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) O[db][r] += v[r] * frr[r];
          if (db % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
      }
      m = M;
      l = Lsum;
    }

    // ---- epilogue: final output + LSE, or a normalized fp32 partial
    if (nsplit <= 1) {
      const int h = h0 + li;
      const bool has_sink = p.sink != nullptr;
      const float s2 = has_sink ? p.sink[h] * kLog2e : kNegInf;
      const float Mx = fmaxf(m, s2);
      float inv, lse2;
      if (Mx == kNegInf) {
        inv = 0.f;
        lse2 = kNegInf;
      } else if (s2 == kPosInf) {
        inv = 0.f;
        lse2 = kPosInf;
      } else {
        const float fo = (m == kNegInf) ? 0.f : fast_exp2(m - Mx);
        const float den = l * fo + (has_sink ? fast_exp2(s2 - Mx) : 0.f);
        inv = den > 0.f ? fo / den : 0.f;
        lse2 = den > 0.f ? Mx + __log2f(den) : kNegInf;
      }
      float ir[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ir[r] = __shfl(inv, 4 * G + r);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint16_t* orow = p.out + (int64_t)t * p.o_st + (int64_t)(h0 + 4 * G + r) * p.o_sh + li;
#pragma unroll
        for (int db = 0; db < 32; ++db) orow[16 * db] = f32_to_bf16_bits(O[db][r] * ir[r]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (G == 0) p.lse[(int64_t)t * p.l_st + h] = (lse2 == kNegInf || lse2 == kPosInf) ? lse2 : lse2 * kLn2;
    } else {
      const int s = s_first + split_k;
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const float lse_p = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
      float ir[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ir[r] = __shfl(inv, 4 * G + r);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* orow = p.o_acc + ((int64_t)s * p.H + h0 + 4 * G + r) * kDv + li;
#pragma unroll
        for (int db = 0; db < 32; ++db) orow[16 * db] = O[db][r] * ir[r];
        __builtin_amdgcn_sched_barrier(0);
      }
      if (G == 0) p.lse_acc[(int64_t)s * p.H + h0 + li] = lse_p;
    }
  }
}

// ---------------------------------------------------------------- combine kernel

__global__ __launch_bounds__(128) void combine_kernel(CombineParams p) {
  const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int s0 = p.num_splits[t];
  const int n = p.num_splits[t + 1] - s0;
  if (n < 2) return;
  const bool has_sink = p.sink != nullptr;
  const float sk = has_sink ? p.sink[h] : kNegInf;
  float M = sk;
  for (int k = 0; k < n; ++k) M = fmaxf(M, p.lse_acc[(int64_t)(s0 + k) * p.H + h]);
  uint16_t* orow = p.out + (int64_t)t * p.o_st + (int64_t)h * p.o_sh + 4 * tid;
  if (M == kNegInf || M == kPosInf) {
    orow[0] = orow[1] = orow[2] = orow[3] = 0;
    if (tid == 0) p.lse[(int64_t)t * p.l_st + h] = M;
    return;
  }
  float den = has_sink ? expf(sk - M) : 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < n; ++k) {
    const float lk = p.lse_acc[(int64_t)(s0 + k) * p.H + h];
    if (lk == kNegInf) continue;
    const float w = expf(lk - M);
    den += w;
    const f32x4 v = *(const f32x4*)(p.o_acc + ((int64_t)(s0 + k) * p.H + h) * kDv + 4 * tid);
    acc += w * v;
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < 4; ++e) orow[e] = f32_to_bf16_bits(acc[e] * inv);
  if (tid == 0) p.lse[(int64_t)t * p.l_st + h] = M + logf(den);
}

// ---------------------------------------------------------------- launchers

hipError_t launch_sched(const SchedParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

template <int NHB, int NRS, int DQK>
static hipError_t launch_decode_t(const DecodeParams& p, int num_parts, int H, int precision, hipStream_t stream) {
  dim3 grid(num_parts, H / (16 * NHB));
  dim3 block(NHB * NRS * 64);
  switch (precision) {
    case 1: hipLaunchKernelGGL((decode_kernel<NHB, NRS, DQK, 1>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((decode_kernel<NHB, NRS, DQK, 3>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                         hipStream_t stream) {
  if (d_qk == 576) {
    switch (heads_per_group) {
      case 16: return launch_decode_t<1, 2, 576>(p, num_parts, p.H, precision, stream);
      default: return launch_decode_t<2, 2, 576>(p, num_parts, p.H, precision, stream);
    }
  }
  switch (heads_per_group) {
    case 16: return launch_decode_t<1, 2, 512>(p, num_parts, p.H, precision, stream);
    default: return launch_decode_t<2, 2, 512>(p, num_parts, p.H, precision, stream);
  }
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(combine_kernel, dim3(p.T, p.H), dim3(kDv / 4), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sda
