// sda_decode_staged.hip -- split-KV decode attention for calls with an NVFP4 list, with FP8_UE8M0 or MODEL1_584
// lists mixed with other formats, or with MODEL1_584 lists at 16 heads per workgroup, on gfx950: records
// staged through registers, widened into a bf16 tile in LDS.
//
// Workgroup = one scheduler part x a group of 16 or 32 query heads, 4 waves. Wave w owns output dims
// [128w, 128w + 128) of every head of the group (its O accumulator: 16-32 heads x 128 dims, fp32).
// A part is a run of (token, 64-position tile) items; each tile is processed as two 32-row sub-tiles.
//
// Pipeline per workgroup, sub-tile k:
//   slot ids of sub-tile k+3 are loaded while sub-tile k computes (they become record addresses at
//   the end of the iteration); the records of sub-tile k+1 are already in flight in registers (issued
//   one iteration earlier, branch-free: masked rows read zeros and their data is zeroed again later).
//   compute(k): QK^T partial over the wave's 128 dims (one dequant scale group) with
//               v_mfma_f32_16x16x32_bf16, KV rows on M, heads on N; partial x that group's scale ->
//               LDS; sum of the four partials; online softmax in base 2 (the reference max moves only
//               when a tile exceeds it by more than 8); O += P' V with P' = p x scale split into NTERM
//               bf16 terms and V read transposed from the tile with ds_read_b64_tr_b16
//   convert(k+1): the staged records -> exact bf16 codes in the row-major LDS tile (rows padded and
//               chunks swizzled against bank conflicts), fp32 scales -> a 32 x 4 LDS table; then the
//               records of k+2 are issued.
// After a token's last sub-tile in the part: the final bf16 output and LSE (sink folded in) when the
// part holds the whole token, otherwise a normalized fp32 partial and its LSE for the combine kernel.
// Sources: masked softmax attention (native_swa_decode.py, _fallback_batched_sdp); gather, validity
// and page addressing (vLLM swapab_decode_attn, stage_inputs); online softmax (native_swa_decode.py,
// BlackwellSWADecodeKernel); swap-AB score product and the sink merge (vLLM swapab_decode_attn,
// device kernel steps 3 and 9); split buffers (FlashMLA sparse_decode.h, o_accum / lse_accum).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sda_device.h"
#include "sda_internal.h"
#include "sda_items.h"

namespace sda {

// The loads a row or a format does not need read these zeros: the data of a masked row is zeroed at
// conversion anyway, but its block scale or exponent is used, and zero bytes give a finite one (the
// cache's own first bytes could read as a NaN scale, and 0 x NaN would reach the tile).
namespace {
__device__ __attribute__((aligned(16))) uint8_t g_zero_staged[64];
}  // namespace

constexpr int KT = 32;    // rows per sub-tile
constexpr int NSLOT = 3;  // address slots: sub-tiles k+1, k+2, k+3

// bf16 tile rows: 1024 bytes of dims and 32 of padding. The LDS serves a 16-byte access of 16 lanes (256
// bytes) per cycle, lanes that fall in the same 4-byte bank at different addresses taking turns; a row
// stride of 1056 bytes puts row r's chunk c at 16-byte slot 2r + c modulo 16, and chunk c of rows with
// bit 3 set is stored at chunk c ^ 1 (tile_swz). Then the QK^T operand reads (one chunk of 16 rows), the
// transposed V reads (8 rows x 2 chunks x 8 bytes per 32 lanes) and the conversion's stores (16 chunks of
// one row, see there) each hit distinct banks, and every offset that varies with the k-step or the dims
// block stays an immediate.
constexpr int kTileRS = 1056;
__device__ __forceinline__ int tile_swz(int r) { return (r >> 3) & 1; }

// Every format this kernel takes holds 512 dims (d_qk = d_v = 512).
template <int NH2>
struct DecodeSmem {
  static constexpr int RS = kTileRS;  // bytes per bf16 row (1024 of dims, then padding)
  char tile[KT * RS];
  f32x4 spart[4][2][NH2][64];  // QK partials [wave][row block][head block][lane]
  float scale[KT][4];          // the four 128-dim scales of each row of the tile (0 = masked row)
  int valid[KT];
  int tile_any;
  uint64_t addr[NSLOT][KT];    // record address per row, 0 = masked
  uint64_t saddr[NSLOT][KT];   // where the row's scales come from (slot scale or the record's fp32 scales)
  int slot_any[NSLOT];
};

// The record loads a build issues besides the four data chunks of each lane: the slot's scale
// (FP8_SLOTSCALE), the four fp32 scales (FP8_528), and for FP8_UE8M0 / MODEL1_584 the exponent word of
// each chunk and MODEL1's bf16 chunks. A call builds the set from its lists' formats; a load the set leaves
// out is not issued at all. Without FP8_UE8M0 / MODEL1_584 lists an NVFP4 lane, which needs two data
// chunks, loads its rows' 16-byte blocks of e4m3 scales into the other two (C4, FP8_528 beside NVFP4: 5
// loads a lane and sub-tile instead of 11).
enum StagedLoads { kLdSlotScale = 1, kLdF32Scales = 2, kLdMx = 4, kLdAll = 7 };

// QR: built for V4.1 calls, whose query dims 448..511 come from the rotated buffer (a separate build, so
// that the extra loads do not add to the register pressure of every other call)
template <int NH2, int NTERM, bool QR, int LS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NH2 == 1 ? 3 : 1)))
void decode_kernel(DecodeParams p) {
  constexpr int RS = DecodeSmem<NH2>::RS;
  __shared__ DecodeSmem<NH2> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int G = lane >> 4, li = lane & 15;
  const int h0 = blockIdx.y * (16 * NH2);

  const ListDev lst0 = p.lst[0];
  const ListDev lst1 = p.lst[p.nlists > 1 ? 1 : 0];
  auto LD = [&](int L) -> const ListDev& { return L ? lst1 : lst0; };
  int32_t mt[SDA_META_INTS];
  part_record(p, mt);
  const int bt = mt[0], bi = mt[1], et = mt[2], ei = mt[3], bk = mt[4];
  if (bt >= p.T || bt > et || (bt == et && bi >= ei)) return;

  // ---- per-lane LDS bases (rows 16 apart have the same swizzle, so every access below is base + a
  // compile-time offset).
  // K operand (k-step ks): row li (+16 rb), chunk 16 w + 4 ks + G at kb + 64 ks. V operand (dims block db):
  // row rv (+16), chunk 16 w + 2 db + cb, bytes 8 (li & 1) .. at vb + 32 db. (The swizzle flips only a
  // chunk's bit 0, which G and cb hold.)
  uint32_t kb, vb;  // byte offsets into sm.tile
  {
    kb = li * RS + 256 * w + 16 * (G ^ tile_swz(li));
    const int rv = 4 * G + (li >> 2);
    const int cb = (li & 3) >> 1;
    vb = rv * RS + 256 * w + 16 * (cb ^ tile_swz(rv)) + 8 * (li & 1);
  }

  // ---- slot ids -> addresses (threads 0..31, one row each)
  int pf_sid = -1;
  auto idx_issue = [&](const Item& it) {
    const int tid = threadIdx.x + opaque_lane_zero();
    pf_sid = -1;
    if (!it.end() && tid < KT) {
      const int pos = it.pos0 + tid;
      if (pos < it.n) pf_sid = LD(it.L).idx[(int64_t)it.t * LD(it.L).row_stride + pos];
    }
  };
  auto idx_finish = [&](const Item& it, int s) {
    if (w == 0) {
      const int tid = threadIdx.x + opaque_lane_zero();
      const ListDev& ld = LD(it.L);
      const bool ok = !it.end() && tid < KT && pf_sid >= 0 && pf_sid < ld.slots;
      uint64_t a = 0, sa = 0;
      if (ok) {
        const uint32_t pg = (uint32_t)pf_sid >> ld.page_shift;
        const uint32_t off = (uint32_t)pf_sid & ((1u << ld.page_shift) - 1u);
        a = (uint64_t)ld.base + (uint64_t)pg * (uint64_t)ld.page_stride + (uint64_t)off * (uint64_t)ld.rec;
        sa = ld.format == SDA_FP8_SLOTSCALE ? (uint64_t)(ld.slot_scale + pf_sid) : a + 512;
      }
      if (tid < KT) {
        sm.addr[s][tid] = a;
        sm.saddr[s][tid] = sa;
      }
      const uint64_t any = __ballot(ok);
      if (tid == 0) sm.slot_any[s] = any != 0 ? 1 : 0;
    }
  };

  // ---- record staging (registers): the sub-tile's data chunks, its scale chunk and bf16 chunk
  // (MODEL1_584 rows: 28 code chunks, then 8 bf16 chunks for dims 448..511, one per lane of 64; the code
  // loads of lanes 28..31 fall inside the record and are not used).
  // The issue is one branch-free sequence of loads, the same for every format of the build's set (LS):
  // a load a row or a format does not need reads g_zero_staged. A load under a format branch would leave
  // its register merged with the value of the previous sub-tile where the branches join, and the
  // compiler's copy there waits for the load, which would stall every sub-tile on a full memory round
  // trip. Registers of loads outside the set hold zero.
  u32x4 stg[4];
  uint32_t stg_sb[4];  // builds with ue8m0 formats: NVFP4 chunks' two e4m3 block scales, or the 16-bit word holding a ue8m0 byte
  uint32_t stg_s1;     // FP8_SLOTSCALE: the row's scale (lanes 0..31)
  u32x4 stg_sc;        // FP8_528 / V32_656: the row's four fp32 scales (lanes 0..31)
  u32x4 stg_rp;
  auto rec_issue = [&](const Item& it, int s) {
    const int tid = threadIdx.x + opaque_lane_zero();
    const ListDev& ld = LD(it.L);
    const uint64_t dummy = (uint64_t)(const void*)g_zero_staged;
    const int fmt = ld.format;
    const bool fp4 = fmt == SDA_NVFP4_288;
    const bool m1 = fmt == SDA_MODEL1_584;
    // ends of the part and all-masked sub-tiles hold zero addresses (every load then reads the zeros)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // builds without ue8m0 or MODEL1 formats: an NVFP4 lane's chunks 2 and 3 take the 16-byte block of
      // scales (bytes 256 + 16 (c / 8) ..) of its rows of chunks 0 and 1, in place of two 16-bit loads
      constexpr bool kScInData = (LS & kLdMx) == 0;
      const int r = fp4 ? (tid >> 4) + 16 * (kScInData ? (k & 1) : k) : (tid >> 5) + 8 * k;
      const int c = fp4 ? tid & 15 : tid & 31;
      const uint64_t a = sm.addr[s][r & (KT - 1)];
      const bool data = a != 0 && (k < 2 || !fp4 || kScInData);
      const int off = (fp4 && k >= 2) ? 256 + 16 * (c >> 3) : 16 * c;
      stg[k] = ld_global_16(data ? a + off : dummy);
      // NVFP4: u16 at byte 256 + 2c. FP8_UE8M0: chunk c (dims 16c .. 16c+15) takes scale byte 512 + c / 2.
      // MODEL1_584: scale byte 576 + c / 4 (64 dims each). Each is read as the aligned 16-bit word holding it.
      const int sb = fp4 ? 256 + 2 * c : fmt == SDA_FP8_UE8M0 ? 512 + ((c >> 1) & ~1) : 576 + ((c >> 2) & ~1);
      const bool sbv = data && (fp4 || fmt == SDA_FP8_UE8M0 || m1);
      if constexpr ((LS & kLdMx) != 0)
        stg_sb[k] = ld_global_u16(sbv ? a + sb : dummy);
      else
        stg_sb[k] = 0u;
    }
    {
      const uint64_t sa = sm.saddr[s][tid & (KT - 1)];
      const bool lo = tid < KT && sa != 0;
      if constexpr ((LS & kLdSlotScale) != 0)
        stg_s1 = *(gbl_u32*)(lo && fmt == SDA_FP8_SLOTSCALE ? sa : dummy);
      else
        stg_s1 = 0u;
      if constexpr ((LS & kLdF32Scales) != 0)
        stg_sc = ld_global_16(lo && (fmt == SDA_FP8_528 || fmt == SDA_V32_656) ? sa : dummy);
      else
        stg_sc = u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr ((LS & kLdMx) != 0) {
      const uint64_t a = sm.addr[s][tid >> 3];
      stg_rp = ld_global_16(a != 0 && m1 ? a + 448 + 16 * (tid & 7) : dummy);
    } else {
      stg_rp = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto rec_convert = [&](const Item& it, int s) {
    const bool live = !it.end() && sm.slot_any[s];
    if (tid == 0) sm.tile_any = live ? 1 : 0;
    if (!live) return;
    const int tid = threadIdx.x + opaque_lane_zero();
    const ListDev& ld = LD(it.L);
    if (ld.format == SDA_NVFP4_288) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int r = (tid >> 4) + 16 * k, c = tid & 15;
        const bool ok = sm.addr[s][r] != 0;
        const u32x4 x = ok ? stg[k] : u32x4{0u, 0u, 0u, 0u};
        uint32_t sbw;
        if constexpr ((LS & kLdMx) != 0) {
          sbw = stg_sb[k];
        } else {  // the chunk's two scale bytes: bytes 2 (c % 8) .. of the row's block of scales
          const u32x4 sv = stg[2 + k];
          const int wi = (c & 7) >> 1;
          const uint32_t wv = (wi & 2) ? ((wi & 1) ? sv[3] : sv[2]) : ((wi & 1) ? sv[1] : sv[0]);
          sbw = wv >> (16 * (c & 1));
        }
        const float s0 = e4m3_to_f32(sbw & 0xFFu), s1 = e4m3_to_f32((sbw >> 8) & 0xFFu);
        const int f = tile_swz(r);
        char* row = sm.tile + r * RS;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // the 16 lanes of row r store output chunks 4c + q together; q rotates with c so that the 16
          // chunks are distinct modulo 16
          const int q = (j + (c >> 1) + (c >> 3)) & 3;
          const uint32_t xq = (q & 2) ? ((q & 1) ? x[3] : x[2]) : ((q & 1) ? x[1] : x[0]);
          const float sc = (q & 2) ? s1 : s0;
          u32x4 o;
          o[0] = e2m1x2_scaled_to_bf16<0>(xq, sc);
          o[1] = e2m1x2_scaled_to_bf16<1>(xq, sc);
          o[2] = e2m1x2_scaled_to_bf16<2>(xq, sc);
          o[3] = e2m1x2_scaled_to_bf16<3>(xq, sc);
          *(u32x4*)(row + 16 * ((4 * c + q) ^ f)) = o;
        }
      }
      if (tid < KT) {
        const float v = sm.addr[s][tid] != 0 ? 1.0f : 0.0f;
        *(f32x4*)sm.scale[tid] = f32x4{v, v, v, v};
      }
    } else {
      const bool ue8m0 = ld.format == SDA_FP8_UE8M0;
      const bool m1 = ld.format == SDA_MODEL1_584;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = (tid >> 5) + 8 * k, c = tid & 31;
        const bool ok = sm.addr[s][r] != 0;
        const u32x4 x = ok ? stg[k] : u32x4{0u, 0u, 0u, 0u};
        // ue8m0 records: the power-of-two scale is applied by the conversion (the row's scale table
        // then holds 1); other formats convert unscaled
        const float cs = ue8m0 ? ue8m0_scale(stg_sb[k] >> (8 * ((c >> 1) & 1)))
                         : m1  ? ue8m0_scale(stg_sb[k] >> (8 * ((c >> 2) & 1)))
                               : 1.0f;
        uint32_t y[8];
        e4m3x4_to_bf16_scaled(x[0], cs, y[0], y[1]);
        e4m3x4_to_bf16_scaled(x[1], cs, y[2], y[3]);
        e4m3x4_to_bf16_scaled(x[2], cs, y[4], y[5]);
        e4m3x4_to_bf16_scaled(x[3], cs, y[6], y[7]);
        if (ue8m0 || m1) {  // scale byte 255 is NaN in the MX encoding: the group's values are NaN
          const bool nan_scale = (__builtin_bit_cast(uint32_t, cs) >> 23) == 255u;
#pragma unroll
          for (int i = 0; i < 8; ++i) y[i] = nan_scale ? 0x7FC07FC0u : y[i];
        }
        const int f = tile_swz(r);
        char* row = sm.tile + r * RS;
        // output chunks 2c and 2c + 1; lanes with c & 8 store the odd one first, so that the 16 chunks of
        // each store are distinct modulo 16
        const bool odd_first = (c & 8) != 0;
        const u32x4 ylo = u32x4{y[0], y[1], y[2], y[3]}, yhi = u32x4{y[4], y[5], y[6], y[7]};
        if (!m1 || c < 28) {  // MODEL1_584: bf16 chunks 56..63 come from the bf16 part below
          *(u32x4*)(row + 16 * ((2 * c + (odd_first ? 1 : 0)) ^ f)) = odd_first ? yhi : ylo;
          *(u32x4*)(row + 16 * ((2 * c + (odd_first ? 0 : 1)) ^ f)) = odd_first ? ylo : yhi;
        }
      }
      if (tid < KT) {
        const bool ok = sm.addr[s][tid] != 0;
        f32x4 sc;
        if (ld.format == SDA_FP8_SLOTSCALE) {
          const float v = __builtin_bit_cast(float, stg_s1);
          sc = f32x4{v, v, v, v};
        } else if (ue8m0 || m1) {
          sc = f32x4{1.f, 1.f, 1.f, 1.f};
        } else {
          sc = __builtin_bit_cast(f32x4, stg_sc);
        }
        *(f32x4*)sm.scale[tid] = ok ? sc : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (m1) {
        const int r = tid >> 3, c = 56 + (tid & 7);
        const bool ok = sm.addr[s][r] != 0;
        *(u32x4*)(sm.tile + r * RS + 16 * (c ^ tile_swz(r))) = ok ? stg_rp : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < KT) sm.valid[tid] = sm.addr[s][tid] != 0 ? 1 : 0;
  };

  // ---- prologue: items k = 0..3, addresses of 0..2, records of 0 converted, records of 1 in flight
  ItemGen gen;
  TokenInfoRegs tinfo;
  gen_init(gen, p, tinfo, mt);
  Item it0 = gen_next<KT>(gen, p, tinfo);
  Item it1 = gen_next<KT>(gen, p, tinfo);
  Item it2 = gen_next<KT>(gen, p, tinfo);
  Item it3 = gen_next<KT>(gen, p, tinfo);
  idx_issue(it0);
  idx_finish(it0, 0);
  idx_issue(it1);
  idx_finish(it1, 1);
  idx_issue(it2);
  idx_finish(it2, 2);
  __syncthreads();
  rec_issue(it0, 0);
  rec_convert(it0, 0);
  rec_issue(it1, 1);
  __syncthreads();

  bf16x8 qreg[NH2][4];
  f32x4 O[NH2][8];
  float m[NH2], l[NH2];
  bool token_start = true;
  int k = 0;

  while (true) {
    if (token_start) {
      const uint16_t* qp = p.q + (int64_t)it0.t * p.q_st + 128 * w + 8 * G;
#pragma unroll
      for (int hb = 0; hb < NH2; ++hb) {
        const uint16_t* qh = qp + (int64_t)(h0 + 16 * hb + li) * p.q_sh;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qreg[hb][ks] = *(const bf16x8*)(qh + 32 * ks);
        if constexpr (QR) {
          // V4.1 calls: dims 448..511 (wave 3, k-steps 2 and 3) from the rotated buffer [T][H][64]; the
          // lane's offset is recomputed here, behind an opaque zero, rather than kept live in the loop
          if (w == 3) {
            const uint16_t* qr =
                p.q_rope + ((int64_t)it0.t * p.H + h0 + 16 * hb) * 64 + (64 * li + 8 * G + opaque_lane_zero());
            qreg[hb][2] = *(const bf16x8*)qr;
            qreg[hb][3] = *(const bf16x8*)(qr + 32);
          }
        }
#pragma unroll
        for (int db = 0; db < 8; ++db) O[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[hb] = kNegInf;
        l[hb] = 0.f;
      }
      token_start = false;
    }
    idx_issue(it3);  // in flight during this sub-tile's compute

    if (sm.tile_any) {
      // ---- QK^T partial over this wave's 128 dims
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4 acc[NH2];
#pragma unroll
        for (int hb = 0; hb < NH2; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 a = *(const bf16x8*)(sm.tile + kb + rb * 16 * RS + 64 * ks);
#pragma unroll
          for (int hb = 0; hb < NH2; ++hb)
            acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[hb][ks], acc[hb], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = sm.scale[rb * 16 + 4 * G + r][w];
#pragma unroll
          for (int hb = 0; hb < NH2; ++hb) acc[hb][r] *= s;
        }
#pragma unroll
        for (int hb = 0; hb < NH2; ++hb) sm.spart[w][rb][hb][lane] = acc[hb];
      }
      __syncthreads();

      // ---- full scores and the online softmax (lane (head li of block hb, G) holds rows 16 rb + 4 G + r)
      float pv[NH2][8];
#pragma unroll
      for (int hb = 0; hb < NH2; ++hb) {
        float z[8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          f32x4 s = sm.spart[0][rb][hb][lane];
#pragma unroll
          for (int ww = 1; ww < 4; ++ww) s += sm.spart[ww][rb][hb][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) z[4 * rb + r] = sm.valid[rb * 16 + 4 * G + r] ? s[r] * p.scale_log2 : kNegInf;
        }
        float tmax = z[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, z[e]);
        tmax = max_across_groups(tmax);
        const bool bump = tmax > m[hb] + 8.0f;
        const float m_new = bump ? tmax : m[hb];
        const float alpha = bump ? fast_exp2(m[hb] - m_new) : 1.0f;
        const float mref = m_new == kNegInf ? 0.f : m_new;  // all rows masked so far: exp2(-inf) = 0
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[hb][e] = fast_exp2(z[e] - mref);
          ps += pv[hb][e];
        }
        l[hb] = l[hb] * alpha + ps;
        m[hb] = m_new;
        if (__any(bump)) {
          float ar[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * G + r);
#pragma unroll
          for (int db = 0; db < 8; ++db) {
#pragma unroll
            for (int r = 0; r < 4; ++r) O[hb][db][r] *= ar[r];
          }
        }
      }

      // ---- O += P' V over this wave's 128 dims
      bf16x8 A[NH2][NTERM];
#pragma unroll
      for (int hb = 0; hb < NH2; ++hb) {
        float pg[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int row = (e < 4) ? 4 * G + e : 16 + 4 * G + (e - 4);
          pg[e] = pv[hb][e] * sm.scale[row][w];
        }
        split_terms<NTERM>(pg, A[hb]);
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const char* v = sm.tile + vb + 32 * db;
        const bf16x4 v0 = lds_read_tr16(v);
        const bf16x4 v1 = lds_read_tr16(v + 16 * RS);
        const bf16x8 B = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int hb = 0; hb < NH2; ++hb) {
#pragma unroll
          for (int t = 0; t < NTERM; ++t)
            O[hb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[hb][t], B, O[hb][db], 0, 0, 0);
        }
      }
    }

    // ---- epilogue after the token's last sub-tile in this part
    if (it1.end() || it1.t != it0.t) {
      const int lane_e = lane + opaque_lane_zero();
      const int li = lane_e & 15, G = lane_e >> 4;
      const int t = it0.t;
      const int s_first = it0.s_first;
      const bool whole = it0.whole && !p.all_partial;
      const int split_k = (t == bt) ? bk : 0;
#pragma unroll
      for (int hb = 0; hb < NH2; ++hb) {
        const float lt = sum_across_groups(l[hb]);
        const int h = h0 + 16 * hb + li;
        float inv, lse_out;
        token_output_factor(m[hb], lt, p.sink != nullptr ? p.sink[h] * kLog2e : kNegInf, whole, inv, lse_out);
        float ir[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ir[r] = __shfl(inv, 4 * G + r);
        if (whole) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            uint16_t* orow = p.out + (int64_t)t * p.o_st + (int64_t)(h0 + 16 * hb + 4 * G + r) * p.o_sh + 128 * w + li;
#pragma unroll
            for (int db = 0; db < 8; ++db) orow[16 * db] = f32_to_bf16_bits(O[hb][db][r] * ir[r]);
          }
          if (w == 0 && G == 0) p.lse[(int64_t)t * p.l_st + h] = lse_out;
        } else {
          const int s = s_first + split_k;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* orow = p.o_acc + ((int64_t)s * p.H + h0 + 16 * hb + 4 * G + r) * kDv + 128 * w + li;
#pragma unroll
            for (int db = 0; db < 8; ++db) orow[16 * db] = O[hb][db][r] * ir[r];
          }
          if (w == 0 && G == 0) p.lse_acc[(int64_t)s * p.H + h] = lse_out;
        }
      }
      token_start = true;
    }
    if (it1.end()) break;

    // ---- next sub-tile: convert its staged records, stage the one after, finish the slot ids of k+3
    __syncthreads();  // the tile and the partials of sub-tile k are no longer read
    rec_convert(it1, (k + 1) % NSLOT);
    rec_issue(it2, (k + 2) % NSLOT);
    idx_finish(it3, (k + 3) % NSLOT);
    it0 = it1;
    it1 = it2;
    it2 = it3;
    it3 = gen_next<KT>(gen, p, tinfo);
    ++k;
    __syncthreads();  // the converted tile and the new addresses are visible
  }
}

template <int NH2, bool QR, int LS>
static hipError_t launch_decode_q(const DecodeParams& p, int num_parts, int precision, hipStream_t stream) {
  dim3 grid(num_parts, p.H / (16 * NH2));
  if (precision == 1)
    hipLaunchKernelGGL((decode_kernel<NH2, 1, QR, LS>), grid, dim3(256), 0, stream, p);
  else if (precision == 2)
    hipLaunchKernelGGL((decode_kernel<NH2, 2, QR, LS>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<NH2, 3, QR, LS>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// The load set of a call: what its lists' formats need. FP8_UE8M0 or MODEL1_584 lists, and V4.1 calls
// (a build of their own), take every load; a call without them has an NVFP4 list and at most one other
// format, and lists of NVFP4 alone take the fp32 scales' set.
static int staged_loads(const DecodeParams& p) {
  int ls = 0;
  for (int L = 0; L < p.nlists; ++L) {
    const int f = p.lst[L].format;
    if (f == SDA_FP8_SLOTSCALE) ls |= kLdSlotScale;
    else if (f == SDA_FP8_528 || f == SDA_V32_656) ls |= kLdF32Scales;
    else if (f != SDA_NVFP4_288) ls |= kLdMx;
  }
  if (p.q_rope || (ls & kLdMx)) return kLdAll;
  return ls == 0 ? kLdF32Scales : ls;
}

template <int NH2>
static hipError_t launch_decode_t(const DecodeParams& p, int num_parts, int precision, hipStream_t stream) {
  if (p.q_rope) return launch_decode_q<NH2, true, kLdAll>(p, num_parts, precision, stream);
  switch (staged_loads(p)) {
    case kLdSlotScale: return launch_decode_q<NH2, false, kLdSlotScale>(p, num_parts, precision, stream);
    case kLdF32Scales: return launch_decode_q<NH2, false, kLdF32Scales>(p, num_parts, precision, stream);
    default: return launch_decode_q<NH2, false, kLdAll>(p, num_parts, precision, stream);
  }
}

// The formats that route here (NVFP4_288, FP8_UE8M0, MODEL1_584, with FP8_SLOTSCALE or FP8_528 beside
// them) all hold 512 dims.
hipError_t launch_decode_staged(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                                hipStream_t stream) {
  if (d_qk != 512) return hipErrorInvalidValue;
  return heads_per_group == 16 ? launch_decode_t<1>(p, num_parts, precision, stream)
                               : launch_decode_t<2>(p, num_parts, precision, stream);
}

}  // namespace sda
