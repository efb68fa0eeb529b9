// sda_decode_ring.hip -- split-KV decode attention over fp8 caches (per-slot scale, 528-byte and
// 656-byte records) for gfx950, with the gathered records streamed into an LDS ring by direct
// global -> LDS loads.
//
// Workgroup = one scheduler part x HS sets of 16 query heads, 4 HS waves; a part is a run of (token,
// 64-row tile) items. The records of a tile land, as raw bytes, in one of NB LDS ring buffers whose
// row stride (528 or 656 bytes) is an odd number of 16-byte chunks, so that consecutive rows start
// in different banks; masked rows (slot -1, out of range, past the length) read a zero record. While
// tile k is computed the records of tiles k+1 .. k+NB-1 are in flight; nothing is staged in registers.
// Every wave gathers 16 / HS rows; wave (head set hs, block wr), tile k:
//   gather: its rows of tile k+NB-1 (global_load_lds_dwordx4, lane-contiguous LDS destinations),
//           after turning their slot ids (loaded one tile earlier) into addresses
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

#include "sda_device.h"
#include "sda_internal.h"
#include "sda_items.h"

namespace sda {

namespace {

// Masked rows gather from here: zero codes and zero scales, so they add nothing to P'V.
__device__ __attribute__((aligned(16))) uint8_t g_zero_record[1024];

}  // namespace

template <int DQK, int HS, int NB>
struct RingSmem {
  static constexpr int RS = DQK == 576 ? 656 : 528;  // ring row stride in bytes (odd number of chunks)
  char ring[NB][kTileRows * RS];
  f32x4 sx[HS][4][64];          // scores of each wave's 16 rows, MFMA output layout
  float sscale[NB][64];         // per-slot scales (FP8_SLOTSCALE)
  float vs[4][64];              // per dim group: its scale for every row of the tile
  uint32_t vmask[NB][4 * HS];   // valid rows of each ring buffer, one mask per gathering wave
  uint64_t raddr[4 * HS][16 / HS];  // per wave: record addresses of the rows it gathers
};

// HS head sets of 16 heads per workgroup (4 HS waves), NB ring buffers (tiles k+1 .. k+NB-1 in flight
// while tile k is computed), NTERM bf16 terms of P'.
template <int DQK, int HS, int NTERM, int NB>
__global__ __launch_bounds__(256 * HS) __attribute__((amdgpu_waves_per_eu(HS == 2 || (DQK == 512 && NB == 2) ? 2 : 1)))
void decode_ring_kernel(DecodeParams p) {
  using Smem = RingSmem<DQK, HS, NB>;
  constexpr int RS = Smem::RS;
  constexpr int RSC = RS / 16;                // chunks per ring row
  constexpr int RW = 16 / HS;                 // rows gathered by each wave
  constexpr int NI = (RW * RSC + 63) / 64;    // gather instructions per wave and tile
  constexpr bool kRope = DQK == 576;
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int hs = w >> 2, wr = w & 3;          // head set; row block (QK^T) and dim group (PV)
  const int G = lane >> 4, li = lane & 15;
  const int h0 = blockIdx.y * (16 * HS) + 16 * hs;  // first head of this wave's set

  // list parameters are read from the kernel arguments where used (scalar loads), not held in registers
  auto LD = [&](int L) -> const ListDev& { return p.lst[L]; };
  const int32_t* mt = p.meta + (int64_t)blockIdx.x * SDA_META_INTS;
  int32_t mrec[SDA_META_INTS];
#pragma unroll
  for (int i = 0; i < SDA_META_INTS; ++i) mrec[i] = mt[i];
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
    for (int j = 0; j < NB; ++j) sids[j] = load_sid(its[j]);  // every slot id load before any gather
#pragma unroll
    for (int j = 0; j + 1 < NB; ++j) {
      if (!its[j].end()) {
        const uint32_t vm = gather(its[j], sids[j], j);
        if (lane == 0) sm.vmask[j][w] = vm;
      }
    }
    sid_next = sids[NB - 1];
  }

  bf16x8 qreg[16];  // k-step 2j: dims 64j + 16G + 0..7, k-step 2j+1: dims 64j + 16G + 8..15
  bf16x8 qrope[2];  // dims 512 + 16G + 0..7 and + 8..15
  auto load_q = [&](int t) {
    const uint16_t* qh = p.q + (int64_t)t * p.q_st + (int64_t)(h0 + li) * p.q_sh + 16 * G;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qreg[2 * j] = *(const bf16x8*)(qh + 64 * j);
      qreg[2 * j + 1] = *(const bf16x8*)(qh + 64 * j + 8);
    }
    if constexpr (kRope) {
      qrope[0] = *(const bf16x8*)(qh + 512);
      qrope[1] = *(const bf16x8*)(qh + 512 + 8);
    }
  };
  load_q(its[0].t);

  f32x4 O[8];
  float m = kNegInf, l = 0.f;
  auto reset_state = [&]() {
#pragma unroll
    for (int db = 0; db < 8; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    if (whole) {
      const float Mx = fmaxf(m, sink2);
      if (Mx == kNegInf) {
        inv = 0.f;
        lse_out = kNegInf;
      } else if (sink2 == kPosInf) {
        inv = 0.f;
        lse_out = kPosInf;
      } else {
        const float fo = (m == kNegInf) ? 0.f : fast_exp2(m - Mx);
        const float den = lt * fo + (sink2 != kNegInf ? fast_exp2(sink2 - Mx) : 0.f);
        inv = den > 0.f ? fo / den : 0.f;
        lse_out = den > 0.f ? (Mx + __log2f(den)) * kLn2 : kNegInf;
      }
    } else {
      inv = lt > 0.f ? 1.0f / lt : 0.f;
      lse_out = lt > 0.f ? (m + __log2f(lt)) * kLn2 : kNegInf;
    }
    float ir[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ir[r] = __shfl(inv, 4 * G + r);
    if (whole) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint16_t* orow = p.out + (int64_t)t * p.o_st + (int64_t)(h0 + 4 * G + r) * p.o_sh + 128 * wr + li;
#pragma unroll
        for (int db = 0; db < 8; ++db) orow[16 * db] = f32_to_bf16_bits(O[db][r] * ir[r]);
      }
      if (wr == 0 && G == 0) p.lse[(int64_t)t * p.l_st + h] = lse_out;
    } else {
      const int s = s_first + split_k;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* orow = p.o_acc + ((int64_t)s * p.H + h0 + 4 * G + r) * kDv + 128 * wr + li;
#pragma unroll
        for (int db = 0; db < 8; ++db) orow[16 * db] = O[db][r] * ir[r];
      }
      if (wr == 0 && G == 0) p.lse_acc[(int64_t)s * p.H + h] = lse_out;
    }
  };

  // per-lane LDS byte offsets within a ring buffer
  const uint32_t qk_off = (uint32_t)((16 * wr + li) * RS + 16 * G);         // + 64 j: dims 64j + 16G ..
  const uint32_t sc_off = (uint32_t)((16 * wr + 4 * G) * RS + 512);         // + r RS: scales of row 16wr+4G+r
  const uint32_t pv_off = (uint32_t)((8 * G + (li >> 1)) * RS + 128 * wr + 8 * (li & 1));  // + 32 kk RS + 16 db
  const uint32_t vs_off = (uint32_t)(lane * RS + 512 + 4 * wr);             // scale of group wr of row `lane`

  // Global operations this wave certainly issued after each gather, for the wait on that gather: the
  // Q loads that follow the gather in its iteration (cnt_tail), and everything of each later
  // iteration (cnt_iter: output stores, the next gather, Q loads). Slot id loads are not counted
  // (a load whose lanes are all masked may be skipped), nor the slot-scale load of a gather, so the
  // counts are lower bounds and the wait never returns early.
  constexpr int QN = kRope ? 18 : 16;  // 16-byte Q loads
  constexpr int SN = 32;               // output stores of an epilogue (per lane: 4 heads x 8 dim blocks)
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
    int c_iter = 0, c_tail = 0;  // this iteration's counts

    if (ep_t >= 0) {
      epilogue(ep_t, ep_s, ep_n);
      reset_state();
      ep_t = -1;
      c_iter += SN;
    }
    // slot ids of tile k+NB, then the gather of tile k+NB-1 into the free buffer
    const int sid_new = load_sid(its[NB]);
    if (!its[NB - 1].end()) {
      const int bg = (k + NB - 1) % NB;
      const uint32_t vm = gather(its[NB - 1], sid_next, bg);
      if (lane == 0) sm.vmask[bg][w] = vm;
      c_iter += NI;
    }
    sid_next = sid_new;

    const Item it0 = its[0], it1 = its[1];
    const ListDev& ld = LD(it0.L);
    const bool slot_scaled = ld.format == SDA_FP8_SLOTSCALE;
    const uint32_t vmw = HS == 1 ? sm.vmask[b][wr] : (sm.vmask[b][2 * wr] | (sm.vmask[b][2 * wr + 1] << 8));
    uint32_t vany = 0;
#pragma unroll
    for (int j = 0; j < 4 * HS; ++j) vany |= sm.vmask[b][j];
    const bool any = vany != 0;
    const char* ring = sm.ring[b];

    if (any) {
      // ---- QK^T for rows 16wr .. 16wr+15
      f32x4 acc[4];
      f32x4 accr = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 lo[4], hi[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 x = *(const u32x4*)(ring + qk_off + 64 * (2 * g + half));
          e4m3x16_to_bf16(x, lo[g], hi[g]);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[g], qreg[2 * (2 * g + half)], acc[g], 0, 0, 0);
#pragma unroll
        for (int g = 0; g < 4; ++g)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[g], qreg[2 * (2 * g + half) + 1], acc[g], 0, 0, 0);
      }
      if constexpr (kRope) {
        const bf16x8 r0 = *(const bf16x8*)(ring + (16 * wr + li) * RS + 528 + 32 * G);
        const bf16x8 r1 = *(const bf16x8*)(ring + (16 * wr + li) * RS + 528 + 32 * G + 16);
        accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0, qrope[0], accr, 0, 0, 0);
        accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r1, qrope[1], accr, 0, 0, 0);
      }
      // fold the rows' scales, mask, write the scores
      f32x4 sc[4];
      if (slot_scaled) {
        const f32x4 ss = *(const f32x4*)&sm.sscale[b][16 * wr + 4 * G];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = f32x4{ss[r], ss[r], ss[r], ss[r]};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = *(const f32x4*)(ring + sc_off + r * RS);
      }
      f32x4 s;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = accr[r];
#pragma unroll
        for (int g = 0; g < 4; ++g) v += acc[g][r] * sc[r][g];
        s[r] = ((vmw >> (4 * G + r)) & 1u) ? v * p.scale_log2 : kNegInf;
      }
      sm.sx[hs][wr][lane] = s;
      // the scale of dim group wr for every row (PV of both head sets)
      if (hs == 0 && !slot_scaled) sm.vs[wr][lane] = *(const float*)(ring + vs_off);
    }
    barrier_lds();  // scores of all rows visible

    // Q of the next tile's token (the registers are free until its QK^T)
    if (!it1.end() && it1.t != it0.t) {
      load_q(it1.t);
      c_iter += QN;
      c_tail = QN;
    }

    if (any) {
      // ---- online softmax; lane (head li, G) holds rows 32 kk + 8 G + e, e = 0..7
      float pv[2][8];
      {
        float z[2][8];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int wv = 2 * kk + (G >> 1);
          const f32x4 a = sm.sx[hs][wv][16 * (2 * (G & 1)) + li];
          const f32x4 c = sm.sx[hs][wv][16 * (2 * (G & 1) + 1) + li];
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
        float ps = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[kk][e] = (m_new == kNegInf) ? 0.f : fast_exp2(z[kk][e] - m_new);
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
          for (int db = 0; db < 8; ++db) {
#pragma unroll
            for (int r = 0; r < 4; ++r) O[db][r] *= ar[r];
          }
        }
      }

      // ---- P' = p x scale (this wave's dim group), split into bf16 terms
      bf16x8 A[2][NTERM];
      {
        const float* vsrc = slot_scaled ? sm.sscale[b] : sm.vs[wr];
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
      }

      // ---- O += P' V over dims 128wr .. 128wr+127, in two halves of 4 dim blocks; the transposed
      // reads of the second half are in flight during the products of the first
      const uint32_t vaddr = lds_u32(ring) + pv_off;
      i32x2 x[2][4][2];
      auto read_half = [&](int half) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) x[half][d][kk] = lds_tr8(vaddr + 32 * kk * RS + 16 * (4 * half + d));
        }
      };
      auto mma_half = [&](int half) {
        bf16x8 B[4][2];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) B[d][kk] = e4m3x8_to_bf16(x[half][d][kk]);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int t = 0; t < NTERM; ++t) {
#pragma unroll
            for (int d = 0; d < 4; ++d)
              O[4 * half + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[kk][t], B[d][kk], O[4 * half + d], 0, 0, 0);
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

    if (it1.end() || it1.t != it0.t) {
      ep_t = it0.t;
      ep_s = it0.s_first;
      ep_n = it0.whole;
    }
    if (it1.end()) break;
#pragma unroll
    for (int r = 0; r + 2 < NB; ++r) {
      cnt_iter[r] = cnt_iter[r + 1];
      cnt_tail[r] = cnt_tail[r + 1];
    }
    cnt_iter[NB - 2] = c_iter;
    cnt_tail[NB - 2] = c_tail;
#pragma unroll
    for (int j = 0; j < NB; ++j) its[j] = its[j + 1];
    its[NB] = gen_next<kTileRows>(gen, p, tinfo);
    ++k;
  }
  if (ep_t >= 0) epilogue(ep_t, ep_s, ep_n);
}

template <int DQK, int HS, int NB>
static hipError_t launch_ring_t(const DecodeParams& p, int num_parts, int precision, hipStream_t stream) {
  dim3 grid(num_parts, p.H / (16 * HS));
  if (precision == 1)
    hipLaunchKernelGGL((decode_ring_kernel<DQK, HS, 1, NB>), grid, dim3(256 * HS), 0, stream, p);
  else if (precision == 2)
    hipLaunchKernelGGL((decode_ring_kernel<DQK, HS, 2, NB>), grid, dim3(256 * HS), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_ring_kernel<DQK, HS, 3, NB>), grid, dim3(256 * HS), 0, stream, p);
  return hipGetLastError();
}

// 16 heads per workgroup: two workgroups per CU, two ring buffers each. 32 heads per workgroup (eight
// waves, one workgroup per CU): three ring buffers.
hipError_t launch_decode_ring(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                              hipStream_t stream) {
  if (d_qk == 576)
    return heads_per_group == 16 ? launch_ring_t<576, 1, 2>(p, num_parts, precision, stream)
                                 : launch_ring_t<576, 2, 3>(p, num_parts, precision, stream);
  return heads_per_group == 16 ? launch_ring_t<512, 1, 2>(p, num_parts, precision, stream)
                               : launch_ring_t<512, 2, 3>(p, num_parts, precision, stream);
}

}  // namespace sda
