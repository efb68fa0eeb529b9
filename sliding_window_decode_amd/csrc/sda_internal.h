// sda_internal.h -- declarations shared by the host API (sda_api.cpp) and the HIP kernels
// (sda_decode_ring.hip, sda_decode_staged.hip, sda_sched.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sda.h"

namespace sda {

constexpr int kTileRows = 64;     // list positions per scheduler tile
constexpr int kDv = 512;          // value dims (the first 512 dims of the latent row)

// One slot list with its cache, in the form the kernels read it.
struct ListDev {
  const int32_t* idx;
  const int32_t* lens;       // nullptr = width
  const uint8_t* base;
  const float* slot_scale;   // FP8_SLOTSCALE only
  int64_t row_stride;
  int64_t page_stride;
  int32_t width;
  int32_t slots;             // num_pages * page_size (< 2^31)
  int32_t page_shift;
  int32_t format;
  int32_t rec;               // record bytes
  int32_t lens_div;          // tokens per length entry (>= 1)
};

struct DecodeParams {
  const uint16_t* q;         // bf16 bits
  int64_t q_st, q_sh;        // element strides
  const uint16_t* q_rope;    // V4.1 calls: dims 448..511 of q after RoPE, [T][H][64]; nullptr: from q
  uint16_t* out;             // bf16 bits
  int64_t o_st, o_sh;
  float* lse;
  int64_t l_st;
  const float* sink;         // [H] or nullptr
  const int32_t* meta;
  const int32_t* num_splits;
  float* o_acc;              // [splits][H][512]
  float* lse_acc;            // [splits][H]
  ListDev lst[2];
  int nlists;
  int T, H;
  float scale_log2;          // softmax scale * log2(e)
  int all_partial;           // every token leaves as an fp32 partial (the combine finishes them all)
};

// The V4.1 call's RoPE inputs (cos_sin row p: cos of pair i at [i], sin at [32 + i]).
struct RopeParams {
  const uint16_t* q;         // bf16 bits, [T][H][512] with strides
  int64_t q_st, q_sh;
  uint16_t* q_out;           // dims 448..511 rotated, [T][H][64] contiguous
  const int64_t* positions;  // [T]
  const float* cos_sin;
  int64_t cs_stride, num_positions;
  int T, H;
};

struct SchedParams {
  const int32_t* lens[2];    // nullptr = width
  int32_t lens_div[2];       // tokens per length entry (>= 1)
  int32_t width[2];
  int nlists;
  int T;
  int num_parts;
  int F;                     // fixed overhead per token, in tiles
  int32_t* meta;
  int32_t* num_splits;
};

struct CombineParams {
  const float* o_acc;
  const float* lse_acc;
  const int32_t* num_splits;
  const float* sink;
  uint16_t* out;
  int64_t o_st, o_sh;
  float* lse;                // nullptr: not written (V4.1 calls only)
  int64_t l_st;
  int T, H;
  // V4.1 output (o8 != nullptr): every token is merged here, its dims 448..511 rotated back and the
  // result cast to MXFP8 (e4m3 codes + one ue8m0 byte per 32 dims) instead of bf16
  const int64_t* positions;
  const float* cos_sin;
  int64_t cs_stride, num_positions;
  uint8_t* o8;
  int64_t o8_st, o8_sh;
  uint8_t* osc;
  int64_t osc_st, osc_sh;
};

// ---------------------------------------------------------------- scheduling math (host + device)
//
// Token t has tiles(t) = max(1, ceil(n_main/64) + ceil(n_extra/64)) tiles, n = clamp(len, 0, width),
// and costs tiles(t) + F. On the cumulative cost axis token t starts at cum(t); its tile i sits at
// cum(t) + F + i and belongs to part floor(position / Q) with Q = ceil(total / num_parts). Parts are
// therefore contiguous ranges of the (token, tile) sequence, in order.

// Clamped length of token t (lens holds one entry per `div` consecutive tokens).
__host__ __device__ inline int clamp_len(const int32_t* lens, int div, int width, int t) {
  int n = lens ? lens[t / div] : width;
  return n < 0 ? 0 : (n > width ? width : n);
}

__host__ __device__ inline int token_tiles(int n0, int n1) {
  int tl = (n0 + kTileRows - 1) / kTileRows + (n1 + kTileRows - 1) / kTileRows;
  return tl < 1 ? 1 : tl;
}

__host__ __device__ inline int64_t part_quantum(int64_t total, int num_parts) {
  int64_t q = (total + num_parts - 1) / num_parts;
  return q < 1 ? 1 : q;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_sched(const SchedParams& p, hipStream_t stream);
// The decode kernels: calls without an NVFP4 list run the ring kernel (sda_decode_ring.hip: records
// streamed into LDS by global -> LDS loads, fp8 widened as read), except mixes of FP8_UE8M0 or
// MODEL1_584 lists with other formats and MODEL1_584 at 16 heads per workgroup; the others the staged kernel
// (sda_decode_staged.hip: records staged in registers and widened once into a bf16 tile; up to three
// workgroups per CU hide the cost of the NVFP4 widening and of the gathers better than one with a deep
// LDS ring); launch_decode (sda_api.cpp) picks one.
hipError_t launch_decode_ring(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                              hipStream_t stream);
hipError_t launch_decode_staged(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                                hipStream_t stream);
// 576-dim records at 64 heads per workgroup (sda_decode_wide.hip: eight waves of 32x32 products, every
// widened operand fragment feeding 32 heads).
hipError_t launch_decode_wide(const DecodeParams& p, int num_parts, int precision, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                         hipStream_t stream);
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
hipError_t launch_rope_q(const RopeParams& p, hipStream_t stream);

}  // namespace sda
