// sda_decode_ring.hip -- split-KV decode attention over fp8 caches (per-slot scale, 528-byte,
// 656-byte and 584-byte MODEL1 records) for gfx950, with the gathered records streamed into an LDS
// ring by direct global -> LDS loads.
//
// Workgroup = one scheduler part x HS sets of 16 query heads, 4 HS waves; a part is a run of (token,
// 64-row tile) items. The records of a tile land, as raw bytes, in one of NB LDS ring buffers whose
// row stride (528 or 656 bytes) is an odd number of 16-byte chunks, so that consecutive rows start
// in different banks; masked rows (slot -1, out of range, past the length) read a zero record. While
// tile k is computed the records of tiles k+1 .. k+NB-1 are in flight; nothing is staged in registers.
// Every wave gathers 16 / HS rows; wave (head set hs, block wr), tile k:
//   gather: its rows of tile k+NB-1 (global_load_lds_dwordx4, lane-contiguous LDS destinations),
//           after turning their slot ids (loaded one tile earlier) into addresses; issued once the
//           scores of tile k are in LDS (the address unit's time overlaps softmax and PV)
//   QK^T:   rows 16wr .. 16wr+15 against the set's heads over all dims, v_mfma_f32_16x16x32_bf16 with
//           rows on M and heads on N; the fp8 codes are widened to bf16 (exactly) as they are read;
//           one accumulator per 128-dim scale group, folded with the rows' scales afterwards
//   scores: through LDS, so that every wave holds all 64 rows of its heads; online softmax in base 2
//           (the reference max moves only when a tile exceeds it by more than 8)
//   PV:     O[:, 128wr .. 128wr+127] += P' V with P' = p x the rows' scale of that dim group split into
//           NTERM bf16 terms, V read transposed with ds_read_b64_tr_b8 and widened to bf16
// A token's output is written once its last tile in the part is done (at the top of the next
// iteration, before that iteration's gather is issued): the final bf16 row and LSE (sink folded in)
// when the part holds the whole token, else a normalized fp32 partial and its LSE for the combine.
//
// Sources: masked softmax attention (native_swa_decode.py, _fallback_batched_sdp); gather, validity
// and page addressing (vLLM swapab_decode_attn, stage_inputs); online softmax (native_swa_decode.py,
// BlackwellSWADecodeKernel); swap-AB score product and the sink merge (vLLM swapab_decode_attn,
// device kernel steps 3 and 9); split buffers (FlashMLA sparse_decode.h, o_accum / lse_accum);
// record layouts (DeepSeek V3.2 / V4 cache formats as described by the vLLM and FlashMLA pages).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sda_device.h"
#include "sda_internal.h"
#include "sda_items.h"

namespace sda {

namespace {

// Masked rows gather from here: zero codes and zero scales, so they add nothing to P'V.
__device__ __attribute__((aligned(16))) uint8_t g_zero_record[1024];

}  // namespace

// Waves of a workgroup with HS head sets: four per set up to 32 heads, eight for 64 heads.
template <int HS>
struct RingShape {
  static constexpr int NW = HS == 4 ? 8 : 4 * HS;  // waves
  static constexpr int WPS = NW / HS;              // waves per head set (4 or 2)
  static constexpr int NRB = 4 / WPS;              // 16-row blocks of a wave's QK^T (1 or 2)
  static constexpr int NDG = 4 / WPS;              // 128-dim groups of a wave's PV (1 or 2)
  static constexpr int RW = kTileRows / NW;        // rows gathered by each wave
  // QK^T: with up to 32 heads a wave takes 16 NRB rows over all dims; with 64 heads the two waves of a
  // head set split the dims instead (all 64 rows, two 128-dim groups and half the rope dims each),
  // which halves the Q registers, and their partial scores are summed when read
  static constexpr bool kDimSplit = HS == 4;
  static constexpr int NPART = kDimSplit ? 2 : 1;  // partial score arrays
};

// Record kinds of a ring kernel build: the fp8 formats with fp32 scales (per slot or per 128 dims), FP8_UE8M0
// (a power-of-two scale per 32 dims) and MODEL1_584 (448 fp8 dims with a power-of-two scale per 64 dims,
// then 64 bf16 dims).
enum RingKind { kRingF32Scales = 0, kRingUe8m0 = 1, kRingModel1 = 2 };

template <int DQK, int HS, int NB, int FK>
struct RingSmem {
  // ring row stride in bytes (odd number of chunks); a MODEL1_584 row holds the record's 576 bytes of
  // codes and bf16 values, then its bytes 568..583 (the scales at row bytes 584..590)
  static constexpr int RS = DQK == 576 ? 656 : (FK == kRingModel1 ? 592 : 528);
  static constexpr int NW = RingShape<HS>::NW;
  char ring[NB][kTileRows * RS];
  f32x4 sx[RingShape<HS>::NPART][HS][4][64];  // (partial) scores per 16-row block and head set, MFMA layout
  float sscale[NB][64];         // per-slot scales (FP8_SLOTSCALE)
  // per scale group: its scale for every row of the tile (128-dim groups; the ue8m0 format's 32-dim
  // groups in the kernels built for it)
  float vs[FK == kRingUe8m0 ? 16 : (FK == kRingModel1 ? 8 : 4)][64];
  uint32_t vmask[NB][NW];       // valid rows of each ring buffer, one mask per gathering wave
  uint64_t raddr[NW][RingShape<HS>::RW];  // per wave: record addresses of the rows it gathers
};

// HS head sets of 16 heads per workgroup (HS = 1, 2, 4: 16, 32 or 64 heads), NB ring buffers (tiles
// k+1 .. k+NB-1 in flight while tile k is computed), NTERM bf16 terms of P'. FK (RingKind): the record
// kind the build decodes; the FP8_UE8M0 and MODEL1_584 builds take calls whose lists are all of that
// format (512 dims), and only them (carrying several decodings raises the register pressure of every
// call; calls that mix them with another format run the staged kernel).
template <int DQK, int HS, int NTERM, int NB, int FK>
__global__ __launch_bounds__(64 * RingShape<HS>::NW)
__attribute__((amdgpu_waves_per_eu(RingShape<HS>::NW == 8 || (DQK == 512 && NB == 2) ? 2 : 1)))
void decode_ring_kernel(DecodeParams p) {
  using Smem = RingSmem<DQK, HS, NB, FK>;
  using Shape = RingShape<HS>;
  constexpr int RS = Smem::RS;
  constexpr int RSC = RS / 16;                // chunks per ring row
  constexpr int RW = Shape::RW;               // rows gathered by each wave
  constexpr int NRB = Shape::NRB, NDG = Shape::NDG;
  constexpr int NI = (RW * RSC + 63) / 64;    // gather instructions per wave and tile
  constexpr bool kRope = DQK == 576;
  constexpr bool kUe8m0 = FK == kRingUe8m0 && DQK == 512;  // FP8_UE8M0 records hold 512 dims
  constexpr bool kM1 = FK == kRingModel1 && DQK == 512;    // MODEL1_584 records
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // w: wave-uniform (scalar)
  const int hs = w / Shape::WPS, sub = w % Shape::WPS;  // head set; its rows (QK^T) and dims (PV)
  const int G = lane >> 4, li = lane & 15;
  const int h0 = blockIdx.y * (16 * HS) + 16 * hs;  // first head of this wave's set

  // list parameters are read from the kernel arguments where used (scalar loads), not held in registers
  auto LD = [&](int L) -> const ListDev& { return p.lst[L]; };
  touch_args(p);
  // A whole-token call (no meta array) knows its token before its lengths arrive: the slot ids of list
  // 0's first NB tiles are loaded first (row min(blockIdx.x, T-1), positions clamped below the width:
  // always readable), and kept for each of the first items that turns out to be that tile. The lengths
  // that follow are scalar loads, so waiting for them does not wait for these.
  const bool spec = p.meta == nullptr;
  int sid_spec[NB];
  {
    const ListDev& l0 = LD(0);
    const int tb = blockIdx.x < (unsigned)p.T ? (int)blockIdx.x : 0;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int pos = kTileRows * j + RW * w + lane % RW;
      sid_spec[j] = l0.idx[(int64_t)tb * l0.row_stride + (pos < l0.width ? pos : l0.width - 1)];
    }
  }
  asm volatile("" ::: "memory");
  int32_t mrec[SDA_META_INTS];
  part_record(p, mrec);
  const int bt = mrec[0], bi = mrec[1], et = mrec[2], ei = mrec[3], bk = mrec[4];
  if (bt >= p.T || bt > et || (bt == et && bi >= ei)) return;

  const float sink2 = p.sink ? p.sink[h0 + li] * kLog2e : kNegInf;  // head li's sink logit, log2 units

  // ---- slot ids -> record addresses, for the RW rows this wave gathers (lane l: row RW w + l % RW)
  auto load_sid = [&](const Item& it) -> int {
    int sid = -1;
    if (!it.end()) {
      const int pos = it.pos0 + RW * w + lane % RW;
      const ListDev& ld = LD(it.L);
      if (pos < it.n) sid = ld.idx[(int64_t)it.t * ld.row_stride + pos];
    }
    return sid;
  };
  const uint64_t zero_rec = (uint64_t)(const void*)g_zero_record;
  // Issues the gather of this wave's rows of item `it` into ring buffer b (NI global -> LDS loads, one
  // more for FP8_SLOTSCALE); returns the wave's valid-row mask.
  auto gather = [&](const Item& it, int sid, int b) -> uint32_t {
    const ListDev& ld = LD(it.L);
    const bool ok = sid >= 0 && sid < ld.slots;
    uint64_t ra = zero_rec, sa = zero_rec;
    if (ok) {
      const uint32_t pg = (uint32_t)sid >> ld.page_shift;
      const uint32_t off = (uint32_t)sid & ((1u << ld.page_shift) - 1u);
      ra = (uint64_t)ld.base + (uint64_t)pg * (uint64_t)ld.page_stride + (uint64_t)off * (uint64_t)ld.rec;
      sa = (uint64_t)(ld.slot_scale + sid);
    }
    const uint32_t vm = (uint32_t)__ballot(ok) & ((1u << RW) - 1u);
    if (lane < RW) sm.raddr[w][lane] = ra;  // read back by the same wave only
    const int nch = ld.rec >> 4;  // chunks in a record (32, 33 or 41)
    char* dst = sm.ring[b] + RW * w * RS;
    // all source addresses first: the compiler keeps LDS reads behind earlier global -> LDS loads.
    // The spare ring chunk of a 512-byte record takes a copy of its chunk 0 (never read); no branch,
    // so that the address reads are not serialized.
    uint64_t src[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = 64 * i + lane;
      const int rl = c / RSC, ch = c - rl * RSC;
      if constexpr (kM1)
        src[i] = sm.raddr[w][rl % RW] + (ch < 36 ? 16 * ch : 568);
      else
        src[i] = sm.raddr[w][rl % RW] + 16 * (ch < nch ? ch : 0);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i < NI - 1 || 64 * i + lane < RW * RSC) dma16(src[i], dst + 1024 * i);
    }
    if (ld.format == SDA_FP8_SLOTSCALE && lane < RW) dma4(sa, &sm.sscale[b][RW * w]);
    return vm;
  };

  // ---- prologue: items k = 0 .. NB, gathers of tiles 0 .. NB-2 in flight, slot ids of tile NB-1
  ItemGen gen;
  TokenInfoRegs tinfo;
  gen_init(gen, p, tinfo, mrec);
  Item its[NB + 1];  // its[j] = tile k + j
#pragma unroll
  for (int j = 0; j <= NB; ++j) its[j] = gen_next<kTileRows>(gen, p, tinfo);
  int sid_next;
  {
    int sids[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {  // every slot id load before any gather
      if (spec && !its[j].end() && its[j].L == 0 && its[j].pos0 == kTileRows * j)
        sids[j] = kTileRows * j + RW * w + lane % RW < its[j].n ? sid_spec[j] : -1;
      else
        sids[j] = load_sid(its[j]);
    }
#pragma unroll
    for (int j = 0; j + 1 < NB; ++j) {
      if (!its[j].end()) {
        const uint32_t vm = gather(its[j], sids[j], j);
        if (lane == 0) sm.vmask[j][w] = vm;
      }
    }
    sid_next = sids[NB - 1];
  }

  // Q of head h0 + li: the 64-dim blocks qj0 .. qj0 + NQJ - 1 (all eight, or the four of this wave's
  // half), k-step 2j: dims 64 (qj0 + j) + 16G + 0..7, k-step 2j+1: + 8..15; rope k-steps qr0 .. (dims
  // 512 + 16G + 8r + 0..7)
  constexpr bool kDimSplit = Shape::kDimSplit;
  constexpr int NQJ = kDimSplit ? 4 : 8;
  constexpr int NQR = kDimSplit ? 1 : 2;
  const int qj0 = kDimSplit ? 4 * sub : 0;
  const int qr0 = kDimSplit ? sub : 0;
  bf16x8 qreg[2 * NQJ];
  bf16x8 qrope[NQR];
  auto load_q = [&](int t) {
    const uint16_t* qh = p.q + (int64_t)t * p.q_st + (int64_t)(h0 + li) * p.q_sh + 16 * G;
#pragma unroll
    for (int j = 0; j < NQJ; ++j) {
      const uint16_t* src = qh + 64 * (qj0 + j);
      if constexpr (DQK == 512) {  // V4.1 calls: the rotated dims 448..511 from their own buffer
        // (the lane's offset is recomputed here, behind an opaque zero, rather than kept live in the loop)
        if (qj0 + j == 7 && p.q_rope)
          src = p.q_rope + ((int64_t)t * p.H + h0) * 64 + (64 * li + 16 * G + opaque_lane_zero());
      }
      qreg[2 * j] = *(const bf16x8*)src;
      qreg[2 * j + 1] = *(const bf16x8*)(src + 8);
    }
    if constexpr (kRope) {
#pragma unroll
      for (int r = 0; r < NQR; ++r) qrope[r] = *(const bf16x8*)(qh + 512 + 8 * (qr0 + r));
    }
  };
  load_q(its[0].t);

  f32x4 O[8 * NDG];  // dims 128 (NDG sub + dg) + 16 db + li of heads h0 + 4G + 0..3
  float m = kNegInf, l = 0.f;
  auto reset_state = [&]() {
#pragma unroll
    for (int db = 0; db < 8 * NDG; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = kNegInf;
    l = 0.f;
  };
  reset_state();

  // ---- output of token t (its last tile in this part is done)
  auto epilogue = [&](int t, int s_first, bool whole) {
    const int split_k = (t == bt) ? bk : 0;
    const float lt = sum_across_groups(l);
    const int h = h0 + li;
    float inv, lse_out;
    token_output_factor(m, lt, sink2, whole, inv, lse_out);
    float ir[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ir[r] = __shfl(inv, 4 * G + r);
    if (whole) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint16_t* orow = p.out + (int64_t)t * p.o_st + (int64_t)(h0 + 4 * G + r) * p.o_sh + 128 * NDG * sub + li;
#pragma unroll
        for (int db = 0; db < 8 * NDG; ++db) orow[16 * db] = f32_to_bf16_bits(O[db][r] * ir[r]);
      }
      if (sub == 0 && G == 0) p.lse[(int64_t)t * p.l_st + h] = lse_out;
    } else {
      const int s = s_first + split_k;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* orow = p.o_acc + ((int64_t)s * p.H + h0 + 4 * G + r) * kDv + 128 * NDG * sub + li;
#pragma unroll
        for (int db = 0; db < 8 * NDG; ++db) orow[16 * db] = O[db][r] * ir[r];
      }
      if (sub == 0 && G == 0) p.lse_acc[(int64_t)s * p.H + h] = lse_out;
    }
  };

  // per-lane LDS byte offsets within a ring buffer; this wave's QK^T rows are the 16-row blocks
  // NRB sub + rb, its PV dims the 128-dim groups NDG sub + dg
  const uint32_t qk_off = (uint32_t)(li * RS + 16 * G);       // + 16 blk RS + 64 j: dims 64j + 16G ..
  const uint32_t sc_off = (uint32_t)(4 * G * RS + 512);       // + 16 blk RS + r RS: scales of row 4G + r
  const uint32_t pv_off = (uint32_t)((8 * G + (li >> 1)) * RS + 128 * NDG * sub + 8 * (li & 1));  // + 32 kk RS + 16 db
  const uint32_t vs_off = (uint32_t)(lane * RS + 512 + 4 * NDG * sub);      // + 4 dg: scale of group NDG sub + dg

  // Global operations this wave certainly issued after each gather, for the wait on that gather: the
  // Q loads that follow the gather in its iteration (cnt_tail: only in the prologue, as a loop iteration
  // issues its gather last), and everything of each later iteration (cnt_iter: output stores, Q loads, the
  // next gather). Slot id loads are not counted
  // (a load whose lanes are all masked may be skipped), nor the slot-scale load of a gather, so the
  // counts are lower bounds and the wait never returns early.
  constexpr int QN = 2 * NQJ + (kRope ? NQR : 0);  // 16-byte Q loads
  constexpr int SN = 32 * NDG;         // output stores of an epilogue (per lane: 4 heads x 8 NDG dim blocks)
  // Entry r of these describes iteration k-NB+1+r (r = 0: the iteration that issued tile k's gather;
  // the prologue counts as iterations -NB+1 .. -1, issuing the gathers of tiles 0 .. NB-2 and then Q).
  int cnt_tail[NB - 1], cnt_iter[NB - 1];
#pragma unroll
  for (int r = 0; r + 1 < NB; ++r) {
    cnt_iter[r] = 0;
    cnt_tail[r] = QN;
#pragma unroll
    for (int i2 = r + 1; i2 + 1 < NB; ++i2) cnt_tail[r] += its[i2].end() ? 0 : NI;
  }

  int k = 0;
  int ep_t = -1, ep_s = 0, ep_n = 1;  // token whose output is pending, its first split, whether whole
  while (true) {
    const int b = k % NB;
    // Tile k landed once this wave has at most as many global ops pending as it issued after the
    // tile's gather (issued in iteration k-NB+1)
    {
      int after = cnt_tail[0];
#pragma unroll
      for (int r = 1; r + 1 < NB; ++r) after += cnt_iter[r];
      vm_wait_atmost(after < 63 ? after : 63);
    }
    barrier_lds();  // every wave's gather of tile k landed; ring buffer (k-1) % NB is free
    int c_iter = 0;  // this iteration's count

    if (ep_t >= 0) {
      epilogue(ep_t, ep_s, ep_n);
      reset_state();
      ep_t = -1;
      c_iter += SN;
    }
    // slot ids of tile k+NB (the gather of tile k+NB-1 into the free buffer follows the scores barrier)
    const int sid_new = load_sid(its[NB]);
    const int sid_g = sid_next;
    sid_next = sid_new;

    const Item it0 = its[0], it1 = its[1];
    const ListDev& ld = LD(it0.L);
    const bool slot_scaled = ld.format == SDA_FP8_SLOTSCALE;
    uint32_t vany = 0;
#pragma unroll
    for (int j = 0; j < Shape::NW; ++j) vany |= sm.vmask[b][j];
    const bool any = vany != 0;
    const char* ring = sm.ring[b];

    if (any) {
      // ---- QK^T for the wave's 16-row blocks (over its 128-dim groups g0 .. g0 + QG - 1)
      constexpr int QRB = kDimSplit ? 4 : NRB;
      constexpr int QG = kDimSplit ? 2 : 4;
      const int g0 = kDimSplit ? 2 * sub : 0;
      // SCALED: FP8_UE8M0 records, whose power-of-two scale of each 32 dims is applied by the conversion
      // (the fold below then multiplies by 1); other formats convert unscaled
      auto qk_blocks = [&](auto ue_tag) {
        constexpr bool SCALED = decltype(ue_tag)::value;
#pragma unroll
        for (int rb = 0; rb < QRB; ++rb) {
          const int blk = kDimSplit ? rb : NRB * sub + rb;  // rows 16 blk .. 16 blk + 15
          // valid rows of the block: gathered by one wave (16 rows each) or two (8 rows each)
          const uint32_t vmw = RW == 16 ? sm.vmask[b][blk] : (sm.vmask[b][2 * blk] | (sm.vmask[b][2 * blk + 1] << 8));
          const uint32_t blk_off = (uint32_t)(16 * blk * RS);
          u32x4 sb = u32x4{0u, 0u, 0u, 0u};  // the row's 16 ue8m0 bytes (MODEL1_584: its 7 in words 0, 1)
          if constexpr (kM1) {
            const u32x2 b8 = *(const u32x2*)(ring + (16 * blk + li) * RS + 584);
            sb = u32x4{b8[0], b8[1], 0u, 0u};
          } else if constexpr (SCALED) {
            sb = *(const u32x4*)(ring + (16 * blk + li) * RS + 512);
          }
          f32x4 acc[QG];
          f32x4 accr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int g = 0; g < QG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 x[QG];
#pragma unroll
            for (int g = 0; g < QG; ++g) x[g] = *(const u32x4*)(ring + qk_off + blk_off + 64 * (2 * (g0 + g) + half));
            // each fragment is widened right before its two products (short-lived temporaries); its 16
            // dims 64 (2 (g0+g) + half) + 16G .. lie in 32-dim group 4 (g0+g) + 2 half + G / 2 (64-dim
            // group 2 (g0+g) + half)
#pragma unroll
            for (int g = 0; g < QG; ++g) {
              const int j64 = 2 * (g0 + g) + half;
              bf16x8 lo, hi;
              if (kM1 && j64 == 7) {  // MODEL1_584 dims 448..511: bf16 values at row byte 448 + 2 (dim - 448)
                const char* rb = ring + qk_off + blk_off - 16 * G + 448 + 32 * G;
                lo = *(const bf16x8*)rb;
                hi = *(const bf16x8*)(rb + 16);
              } else {
                const float cs = kM1 ? ue8m0_scale(sb[j64 >> 2] >> (8 * (j64 & 3)))
                                 : SCALED ? ue8m0_scale(sb[g0 + g] >> (8 * (2 * half + (G >> 1)))) : 1.0f;
                e4m3x16_to_bf16_scaled(x[g], cs, lo, hi);
              }
              acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, qreg[2 * (2 * g + half)], acc[g], 0, 0, 0);
              acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, qreg[2 * (2 * g + half) + 1], acc[g], 0, 0, 0);
            }
          }
          if constexpr (kRope) {
            const char* rr = ring + (16 * blk + li) * RS + 528 + 32 * G + 16 * qr0;
#pragma unroll
            for (int r = 0; r < NQR; ++r)
              accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(rr + 16 * r), qrope[r], accr, 0, 0, 0);
          }
          // fold the rows' scales, mask, write the (partial) scores
          f32x4 sc[4];
          if (slot_scaled) {
            const f32x4 ss = *(const f32x4*)&sm.sscale[b][16 * blk + 4 * G];
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[r] = f32x4{ss[r], ss[r], ss[r], ss[r]};
          } else if (SCALED || kM1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[r] = f32x4{1.f, 1.f, 1.f, 1.f};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[r] = *(const f32x4*)(ring + sc_off + blk_off + r * RS);
          }
          f32x4 s;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = accr[r];
#pragma unroll
            for (int g = 0; g < QG; ++g) v += acc[g][r] * sc[r][g0 + g];
            s[r] = ((vmw >> (4 * G + r)) & 1u) ? v * p.scale_log2 : kNegInf;
          }
          sm.sx[kDimSplit ? sub : 0][hs][blk][lane] = s;
        }
      };
      if constexpr (kUe8m0)
        qk_blocks(std::true_type{});
      else
        qk_blocks(std::false_type{});
      // the scale of each of this wave's dim groups for every row (PV of all head sets)
      if (hs == 0 && !slot_scaled) {
        if constexpr (kM1) {
#pragma unroll
          for (int dg = 0; dg < NDG; ++dg) {  // the group's two 64-dim scales (the bf16 dims: 1)
            const int gi = NDG * sub + dg;
            const uint32_t wd = *(const uint16_t*)(ring + lane * RS + 584 + 2 * gi);
            sm.vs[2 * gi][lane] = ue8m0_value(wd);
            sm.vs[2 * gi + 1][lane] = gi == 3 ? 1.0f : ue8m0_value(wd >> 8);
          }
        } else if constexpr (kUe8m0) {
#pragma unroll
          for (int dg = 0; dg < NDG; ++dg) {
            const uint32_t wd = *(const uint32_t*)(ring + vs_off + 4 * dg);  // the group's 4 ue8m0 bytes
#pragma unroll
            for (int sg = 0; sg < 4; ++sg) sm.vs[4 * (NDG * sub + dg) + sg][lane] = ue8m0_value(wd >> (8 * sg));
          }
        } else {
#pragma unroll
          for (int dg = 0; dg < NDG; ++dg) sm.vs[NDG * sub + dg][lane] = *(const float*)(ring + vs_off + 4 * dg);
        }
      }
    }
    barrier_lds();  // scores of all rows visible

    // Q of the next tile's token (the registers are free until its QK^T)
    if (!it1.end() && it1.t != it0.t) {
      load_q(it1.t);
      c_iter += QN;
    }
    // the gather of tile k+NB-1 into the free buffer: the last global operation of the iteration, issued
    // after QK^T so that the address unit's time overlaps softmax and PV
    if (!its[NB - 1].end()) {
      const int bg = (k + NB - 1) % NB;
      const uint32_t vm = gather(its[NB - 1], sid_g, bg);
      if (lane == 0) sm.vmask[bg][w] = vm;
      c_iter += NI;
    }

    if (any) {
      // ---- online softmax; lane (head li, G) holds rows 32 kk + 8 G + e, e = 0..7
      float pv[2][8];
      {
        float z[2][8];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int wv = 2 * kk + (G >> 1);
          f32x4 a = sm.sx[0][hs][wv][16 * (2 * (G & 1)) + li];
          f32x4 c = sm.sx[0][hs][wv][16 * (2 * (G & 1) + 1) + li];
          if constexpr (kDimSplit) {  // the other half's partial scores (a masked row is -inf in both)
            a += sm.sx[1][hs][wv][16 * (2 * (G & 1)) + li];
            c += sm.sx[1][hs][wv][16 * (2 * (G & 1) + 1) + li];
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            z[kk][r] = a[r];
            z[kk][4 + r] = c[r];
          }
        }
        float tmax = z[0][0];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, z[kk][e]);
        }
        tmax = max_across_groups(tmax);
        const bool bump = tmax > m + 8.0f;
        const float m_new = bump ? tmax : m;
        const float alpha = bump ? fast_exp2(m - m_new) : 1.0f;
        const float mref = m_new == kNegInf ? 0.f : m_new;  // all rows masked so far: exp2(-inf) = 0
        float ps = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[kk][e] = fast_exp2(z[kk][e] - mref);
            ps += pv[kk][e];
          }
        }
        l = l * alpha + ps;
        m = m_new;
        if (__any(bump)) {
          float ar[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * G + r);
#pragma unroll
          for (int db = 0; db < 8 * NDG; ++db) {
#pragma unroll
            for (int r = 0; r < 4; ++r) O[db][r] *= ar[r];
          }
        }
      }

      // ---- per dim group of this wave: P' = p x the rows' scale of the group, split into bf16 terms;
      // O += P' V over its 128 dims in two halves of 4 dim blocks (the transposed reads of the second
      // half are in flight during the products of the first). FP8_UE8M0: one P' per 32 dims, in four
      // quarters of 2 dim blocks.
      auto make_p = [&](const float* vsrc, bf16x8 (&A)[2][NTERM]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const f32x4 a = *(const f32x4*)(vsrc + 32 * kk + 8 * G);
          const f32x4 c = *(const f32x4*)(vsrc + 32 * kk + 8 * G + 4);
          float pg[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pg[r] = pv[kk][r] * a[r];
            pg[4 + r] = pv[kk][4 + r] * c[r];
          }
          split_terms<NTERM>(pg, A[kk]);
        }
      };
#pragma unroll
      for (int dg = 0; dg < NDG; ++dg) {
        const uint32_t vaddr = lds_u32(ring) + pv_off + 128 * dg;
        if constexpr (kM1) {
          // MODEL1_584: one P' per 64 dims, in four quarters of 2 dim blocks; the last two quarters of
          // dim group 3 (dims 448..511) are bf16 values, read transposed 16 bits at a time: lane (li, G)
          // points at row 32 kk + 8 G + li / 4 (+ 4), dims 16 li % 4 .. + 3 of its block, and receives
          // dim li of the group's four rows
          const int gi = NDG * sub + dg;
          const uint32_t baddr = lds_u32(ring) + (uint32_t)((8 * G + (li >> 2)) * RS + 448 + 8 * (li & 3));
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            bf16x8 A[2][NTERM];
            make_p(sm.vs[2 * gi + h2], A);
            if (gi == 3 && h2 == 1) {
              i32x2 y[4][2][2];  // [dim block][kk][rows +0 / +4]
#pragma unroll
              for (int d = 0; d < 4; ++d) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                  y[d][kk][0] = lds_tr16(baddr + 32 * kk * RS + 32 * d);
                  y[d][kk][1] = lds_tr16(baddr + (32 * kk + 4) * RS + 32 * d);
                }
              }
              asm volatile("s_waitcnt lgkmcnt(0)"
                           : "+v"(y[0][0][0]), "+v"(y[0][0][1]), "+v"(y[0][1][0]), "+v"(y[0][1][1]),
                             "+v"(y[1][0][0]), "+v"(y[1][0][1]), "+v"(y[1][1][0]), "+v"(y[1][1][1]),
                             "+v"(y[2][0][0]), "+v"(y[2][0][1]), "+v"(y[2][1][0]), "+v"(y[2][1][1]),
                             "+v"(y[3][0][0]), "+v"(y[3][0][1]), "+v"(y[3][1][0]), "+v"(y[3][1][1]));
#pragma unroll
              for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                  const bf16x8 B = __builtin_bit_cast(
                      bf16x8, u32x4{(uint32_t)y[d][kk][0][0], (uint32_t)y[d][kk][0][1], (uint32_t)y[d][kk][1][0],
                                    (uint32_t)y[d][kk][1][1]});
                  f32x4& o = O[8 * dg + 4 + d];
#pragma unroll
                  for (int t = 0; t < NTERM; ++t) o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kk][t], B, o, 0, 0, 0);
                }
              }
              continue;
            }
            i32x2 x[4][2];  // [dim block][kk]
#pragma unroll
            for (int d = 0; d < 4; ++d) {
#pragma unroll
              for (int kk = 0; kk < 2; ++kk) x[d][kk] = lds_tr8(vaddr + 32 * kk * RS + 16 * (4 * h2 + d));
            }
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[1][0]), "+v"(x[1][1]), "+v"(x[2][0]),
                           "+v"(x[2][1]), "+v"(x[3][0]), "+v"(x[3][1]));
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const bf16x8 B = e4m3x8_to_bf16(x[d][kk]);
                f32x4& o = O[8 * dg + 4 * h2 + d];
#pragma unroll
                for (int t = 0; t < NTERM; ++t) o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kk][t], B, o, 0, 0, 0);
              }
            }
          }
          continue;
        }
        if constexpr (kUe8m0) {
          i32x2 x[2][2][2];  // [buffer][dim block of the quarter][kk]
          auto read_q = [&](int sg, int buf) {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
#pragma unroll
              for (int kk = 0; kk < 2; ++kk) x[buf][d][kk] = lds_tr8(vaddr + 32 * kk * RS + 16 * (2 * sg + d));
            }
          };
          read_q(0, 0);
#pragma unroll
          for (int sg = 0; sg < 4; ++sg) {
            const int buf = sg & 1;
            bf16x8 A[2][NTERM];
            make_p(sm.vs[4 * (NDG * sub + dg) + sg], A);
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(x[buf][0][0]), "+v"(x[buf][0][1]), "+v"(x[buf][1][0]), "+v"(x[buf][1][1]));
            if (sg < 3) read_q(sg + 1, buf ^ 1);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
              for (int d = 0; d < 2; ++d) {
                const bf16x8 B = e4m3x8_to_bf16(x[buf][d][kk]);
                f32x4& o = O[8 * dg + 2 * sg + d];
#pragma unroll
                for (int t = 0; t < NTERM; ++t) o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kk][t], B, o, 0, 0, 0);
              }
            }
          }
          continue;
        }
        bf16x8 A[2][NTERM];
        make_p(slot_scaled ? sm.sscale[b] : sm.vs[NDG * sub + dg], A);
        i32x2 x[2][4][2];
        auto read_half = [&](int half) {
#pragma unroll
          for (int d = 0; d < 4; ++d) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) x[half][d][kk] = lds_tr8(vaddr + 32 * kk * RS + 16 * (4 * half + d));
          }
        };
        auto mma_half = [&](int half) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const bf16x8 B = e4m3x8_to_bf16(x[half][d][kk]);
              f32x4& o = O[8 * dg + 4 * half + d];
#pragma unroll
              for (int t = 0; t < NTERM; ++t) o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kk][t], B, o, 0, 0, 0);
            }
          }
        };
        read_half(0);
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(x[0][0][0]), "+v"(x[0][0][1]), "+v"(x[0][1][0]), "+v"(x[0][1][1]), "+v"(x[0][2][0]),
                       "+v"(x[0][2][1]), "+v"(x[0][3][0]), "+v"(x[0][3][1]));
        read_half(1);
        mma_half(0);
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(x[1][0][0]), "+v"(x[1][0][1]), "+v"(x[1][1][0]), "+v"(x[1][1][1]), "+v"(x[1][2][0]),
                       "+v"(x[1][2][1]), "+v"(x[1][3][0]), "+v"(x[1][3][1]));
        mma_half(1);
      }
    }

    if (it1.end() || it1.t != it0.t) {
      ep_t = it0.t;
      ep_s = it0.s_first;
      ep_n = it0.whole && !p.all_partial;
    }
    if (it1.end()) break;
#pragma unroll
    for (int r = 0; r + 2 < NB; ++r) {
      cnt_iter[r] = cnt_iter[r + 1];
      cnt_tail[r] = cnt_tail[r + 1];
    }
    cnt_iter[NB - 2] = c_iter;
    cnt_tail[NB - 2] = 0;
#pragma unroll
    for (int j = 0; j < NB; ++j) its[j] = its[j + 1];
    its[NB] = gen_next<kTileRows>(gen, p, tinfo);
    ++k;
  }
  if (ep_t >= 0) epilogue(ep_t, ep_s, ep_n);
}

template <int DQK, int HS, int NB, int FK>
static hipError_t launch_ring_t(const DecodeParams& p, int num_parts, int precision, hipStream_t stream) {
  dim3 grid(num_parts, p.H / (16 * HS));
  const dim3 block(64 * RingShape<HS>::NW);
  if (precision == 1)
    hipLaunchKernelGGL((decode_ring_kernel<DQK, HS, 1, NB, FK>), grid, block, 0, stream, p);
  else if (precision == 2)
    hipLaunchKernelGGL((decode_ring_kernel<DQK, HS, 2, NB, FK>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_ring_kernel<DQK, HS, 3, NB, FK>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int DQK, int HS, int NB>
static hipError_t launch_ring_any(const DecodeParams& p, int num_parts, int precision, int kind, hipStream_t stream) {
  if constexpr (DQK == 512) {
    if (kind == kRingUe8m0) return launch_ring_t<DQK, HS, NB, kRingUe8m0>(p, num_parts, precision, stream);
    if constexpr (HS > 1) {  // 592-byte ring rows: two buffers of 64 rows leave no room for a second workgroup
      if (kind == kRingModel1) return launch_ring_t<DQK, HS, NB, kRingModel1>(p, num_parts, precision, stream);
    }
  }
  return launch_ring_t<DQK, HS, NB, kRingF32Scales>(p, num_parts, precision, stream);
}

// 16 heads per workgroup: two workgroups per CU, two ring buffers each. 32 heads (eight waves, one
// workgroup per CU): three ring buffers. 64 heads (eight waves with twice the rows and dims each):
// three ring buffers, every record gathered once per 64 heads. Every list must be of the kind the
// build takes: FP8_UE8M0 lists only with one another, MODEL1_584 lists likewise and with 32 or more
// heads per workgroup (launch_decode sends other mixes to the staged kernel).
hipError_t launch_decode_ring(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                              hipStream_t stream) {
  const int kind = p.lst[0].format == SDA_FP8_UE8M0 ? kRingUe8m0
                   : p.lst[0].format == SDA_MODEL1_584 ? kRingModel1 : kRingF32Scales;
  if (d_qk == 576) {  // 64 heads of 576-dim records run the wide kernel
    if (heads_per_group == 16) return launch_ring_any<576, 1, 2>(p, num_parts, precision, kRingF32Scales, stream);
    if (heads_per_group == 32) return launch_ring_any<576, 2, 3>(p, num_parts, precision, kRingF32Scales, stream);
    return hipErrorInvalidValue;
  }
  if (heads_per_group == 16) {
    if (kind == kRingModel1) return hipErrorInvalidValue;
    return launch_ring_any<512, 1, 2>(p, num_parts, precision, kind, stream);
  }
  if (heads_per_group == 32) return launch_ring_any<512, 2, 3>(p, num_parts, precision, kind, stream);
  return launch_ring_any<512, 4, 3>(p, num_parts, precision, kind, stream);
}

}  // namespace sda
