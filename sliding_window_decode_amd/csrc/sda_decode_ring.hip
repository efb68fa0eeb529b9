// sda_decode_ring.hip -- split-KV decode attention over fp8 caches (per-slot scale, 528-byte and
// 656-byte records) for gfx950, with the gathered records streamed into an LDS ring by direct
// global -> LDS loads.
//
// Workgroup = one scheduler part x a group of 16 NH2 query heads, 4 waves; a part is a run of (token,
// 64-row tile) items. The records of a tile land, as raw bytes, in one of two LDS ring buffers whose
// row stride (528 or 656 bytes) is an odd number of 16-byte chunks, so that consecutive rows start
// in different banks; masked rows (slot -1, out of range, past the length) read a zero record. While
// tile k is computed the records of tile k+1 are in flight, and nothing is staged in registers.
// Wave w, tile k:
//   gather: the records of rows 16w .. 16w+15 of tile k+1 (global_load_lds_dwordx4, lane-contiguous
//           LDS destinations), after turning their slot ids (loaded one tile earlier) into addresses
//   QK^T:   rows 16w .. 16w+15 against the group's heads over all dims, v_mfma_f32_16x16x32_bf16 with
//           rows on M and heads on N; the fp8 codes are widened to bf16 (exactly) as they are read;
//           one accumulator per 128-dim scale group, folded with the rows' scales afterwards
//   scores: through LDS, so that every wave holds all 64 rows of its heads; online softmax in base 2
//           (the reference max moves only when a tile exceeds it by more than 8)
//   PV:     O[:, 128w .. 128w+127] += P' V with P' = p x the rows' scale of that dim group split into
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

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void gbl_void;
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Masked rows gather from here: zero codes and zero scales, so they add nothing to P'V.
__device__ __attribute__((aligned(16))) uint8_t g_zero_record[1024];

__device__ __forceinline__ void dma16(uint64_t src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)(uintptr_t)src, (lds_void*)lds_wave_base, 16, 0, 0);
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
// result may only be used after lds_wait().
__device__ __forceinline__ i32x2 lds_tr8(uint32_t lds_addr) {
  i32x2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(r) : "v"(lds_addr));
  return r;
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 e4m3 codes -> two bf16x8 (codes 0..7, 8..15), exact.
__device__ __forceinline__ void e4m3x16_to_bf16(const u32x4 x, bf16x8& lo, bf16x8& hi) {
  uint32_t y[8];
  e4m3x4_to_bf16(x[0], y[0], y[1]);
  e4m3x4_to_bf16(x[1], y[2], y[3]);
  e4m3x4_to_bf16(x[2], y[4], y[5]);
  e4m3x4_to_bf16(x[3], y[6], y[7]);
  lo = __builtin_bit_cast(bf16x8, u32x4{y[0], y[1], y[2], y[3]});
  hi = __builtin_bit_cast(bf16x8, u32x4{y[4], y[5], y[6], y[7]});
}

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(const i32x2 x) {
  uint32_t y[4];
  e4m3x4_to_bf16((uint32_t)x[0], y[0], y[1]);
  e4m3x4_to_bf16((uint32_t)x[1], y[2], y[3]);
  return __builtin_bit_cast(bf16x8, u32x4{y[0], y[1], y[2], y[3]});
}

}  // namespace

template <int DQK, int NH2>
struct RingSmem {
  static constexpr int RS = DQK == 576 ? 656 : 528;  // ring row stride in bytes (odd number of chunks)
  char ring[2][kTileRows * RS];
  f32x4 sx[4][NH2][64];   // scores of each wave's 16 rows, MFMA output layout
  float sscale[2][64];    // per-slot scales (FP8_SLOTSCALE)
  float vs[4][64];        // per wave: the scale of its dim group for every row of the tile
  uint32_t vmask[2][4];   // valid rows of each ring buffer, 16 bits per wave
  uint64_t raddr[4][16];  // per wave: record addresses of its rows of the tile being gathered
};

template <int DQK, int NH2, int NTERM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DQK == 512 && NH2 == 1 ? 2 : 1)))
void decode_ring_kernel(DecodeParams p) {
  using Smem = RingSmem<DQK, NH2>;
  constexpr int RS = Smem::RS;
  constexpr int RSC = RS / 16;                // chunks per ring row
  constexpr int NI = (16 * RSC + 63) / 64;    // gather instructions per wave and tile
  constexpr bool kRope = DQK == 576;
  __shared__ Smem sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int G = lane >> 4, li = lane & 15;
  const int h0 = blockIdx.y * (16 * NH2);

  const ListDev lst0 = p.lst[0];
  const ListDev lst1 = p.lst[p.nlists > 1 ? 1 : 0];
  auto LD = [&](int L) -> const ListDev& { return L ? lst1 : lst0; };
  const int32_t* mt = p.meta + (int64_t)blockIdx.x * SDA_META_INTS;
  const int bt = mt[0], bi = mt[1], et = mt[2], ei = mt[3], bk = mt[4];
  if (bt >= p.T || bt > et || (bt == et && bi >= ei)) return;

  float sink2[NH2];  // sink logit of head li of each head block, in log2 units
#pragma unroll
  for (int hb = 0; hb < NH2; ++hb) sink2[hb] = p.sink ? p.sink[h0 + 16 * hb + li] * kLog2e : kNegInf;

  // ---- slot ids -> record addresses for this wave's 16 rows (lane l: row 16w + l % 16)
  auto load_sid = [&](const Item& it) -> int {
    int sid = -1;
    if (!it.end) {
      const int pos = it.pos0 + 16 * w + li;
      const ListDev& ld = LD(it.L);
      if (pos < it.n) sid = ld.idx[(int64_t)it.t * ld.row_stride + pos];
    }
    return sid;
  };
  const uint64_t zero_rec = (uint64_t)(const void*)g_zero_record;
  // Issues the gather of this wave's rows of item `it` into ring buffer b; returns the wave's 16-bit
  // valid mask.
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
    const uint32_t vm = (uint32_t)__ballot(ok) & 0xFFFFu;
    if (lane < 16) sm.raddr[w][lane] = ra;  // read back by the same wave only
    const int nch = ld.rec >> 4;  // chunks in a record (32, 33 or 41)
    char* dst = sm.ring[b] + 16 * w * RS;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = 64 * i + lane;
      const int rl = c / RSC, ch = c - rl * RSC;
      const uint64_t a = sm.raddr[w][rl & 15];
      const uint64_t src = ch < nch ? a + 16 * ch : zero_rec;  // spare chunk of a 512-byte record
      if (i < NI - 1 || c < 16 * RSC) dma16(src, dst + 1024 * i);
    }
    if (ld.format == SDA_FP8_SLOTSCALE && lane < 16) dma4(sa, &sm.sscale[b][16 * w]);
    return vm;
  };

  // ---- prologue: gather of item 0 in flight, slot ids of item 1 loaded, Q of item 0 loaded
  ItemGen gen;
  gen_init(gen, p, bt, bi, et, ei);
  Item it0 = gen_next<kTileRows>(gen, p);
  Item it1 = gen_next<kTileRows>(gen, p);
  Item it2 = gen_next<kTileRows>(gen, p);
  {
    const int sid0 = load_sid(it0);
    const uint32_t vm = gather(it0, sid0, 0);
    if (lane == 0) sm.vmask[0][w] = vm;
  }
  int sid = load_sid(it1);

  bf16x8 qreg[NH2][16];  // k-step 2j: dims 64j + 16G + 0..7, k-step 2j+1: dims 64j + 16G + 8..15
  bf16x8 qrope[NH2][2];  // dims 512 + 16G + 0..7 and + 8..15
  auto load_q = [&](int t) {
#pragma unroll
    for (int hb = 0; hb < NH2; ++hb) {
      const uint16_t* qh = p.q + (int64_t)t * p.q_st + (int64_t)(h0 + 16 * hb + li) * p.q_sh + 16 * G;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qreg[hb][2 * j] = *(const bf16x8*)(qh + 64 * j);
        qreg[hb][2 * j + 1] = *(const bf16x8*)(qh + 64 * j + 8);
      }
      if constexpr (kRope) {
        qrope[hb][0] = *(const bf16x8*)(qh + 512);
        qrope[hb][1] = *(const bf16x8*)(qh + 512 + 8);
      }
    }
  };
  load_q(it0.t);

  f32x4 O[NH2][8];
  float m[NH2], l[NH2];
  auto reset_state = [&]() {
#pragma unroll
    for (int hb = 0; hb < NH2; ++hb) {
#pragma unroll
      for (int db = 0; db < 8; ++db) O[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[hb] = kNegInf;
      l[hb] = 0.f;
    }
  };
  reset_state();

  // ---- output of token t (its last tile in this part is done)
  auto epilogue = [&](int t, int s_first, int nsplit) {
    const int split_k = (t == bt) ? bk : 0;
#pragma unroll
    for (int hb = 0; hb < NH2; ++hb) {
      const float lt = sum_across_groups(l[hb]);
      const int h = h0 + 16 * hb + li;
      float inv, lse_out;
      if (nsplit <= 1) {
        const float s2 = sink2[hb];
        const float Mx = fmaxf(m[hb], s2);
        if (Mx == kNegInf) {
          inv = 0.f;
          lse_out = kNegInf;
        } else if (s2 == kPosInf) {
          inv = 0.f;
          lse_out = kPosInf;
        } else {
          const float fo = (m[hb] == kNegInf) ? 0.f : fast_exp2(m[hb] - Mx);
          const float den = lt * fo + (s2 != kNegInf ? fast_exp2(s2 - Mx) : 0.f);
          inv = den > 0.f ? fo / den : 0.f;
          lse_out = den > 0.f ? (Mx + __log2f(den)) * kLn2 : kNegInf;
        }
      } else {
        inv = lt > 0.f ? 1.0f / lt : 0.f;
        lse_out = lt > 0.f ? (m[hb] + __log2f(lt)) * kLn2 : kNegInf;
      }
      float ir[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ir[r] = __shfl(inv, 4 * G + r);
      if (nsplit <= 1) {
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
  };

  // per-lane LDS byte offsets within a ring buffer
  const uint32_t qk_off = (uint32_t)((16 * w + li) * RS + 16 * G);         // + 64 j: dims 64j + 16G ..
  const uint32_t sc_off = (uint32_t)((16 * w + 4 * G) * RS + 512);         // + r RS: scales of row 16w+4G+r
  const uint32_t pv_off = (uint32_t)((8 * G + (li >> 1)) * RS + 128 * w + 8 * (li & 1));  // + 32 kk RS + 16 db
  const uint32_t vs_off = (uint32_t)(lane * RS + 512 + 4 * w);             // scale of group w of row `lane`

  int k = 0;
  int ep_t = -1, ep_s = 0, ep_n = 0;  // token whose output is pending, its split range
  while (true) {
    const int b = k & 1;
    // gather of tile k landed: drain this wave's loads, then the barrier (ring buffer b^1 is free)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    if (ep_t >= 0) {
      epilogue(ep_t, ep_s, ep_n);
      reset_state();
      ep_t = -1;
    }
    // gather of tile k+1 into the free buffer, slot ids of tile k+2
    if (!it1.end) {
      const uint32_t vm = gather(it1, sid, b ^ 1);
      if (lane == 0) sm.vmask[b ^ 1][w] = vm;
    }
    sid = load_sid(it2);

    const ListDev& ld = LD(it0.L);
    const bool slot_scaled = ld.format == SDA_FP8_SLOTSCALE;
    const uint32_t vmw = sm.vmask[b][w];
    const bool any = (sm.vmask[b][0] | sm.vmask[b][1] | sm.vmask[b][2] | sm.vmask[b][3]) != 0;
    const char* ring = sm.ring[b];

    if (any) {
      // ---- QK^T for rows 16w .. 16w+15
      f32x4 acc[NH2][4];
      f32x4 accr[NH2];
#pragma unroll
      for (int hb = 0; hb < NH2; ++hb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) acc[hb][g] = f32x4{0.f, 0.f, 0.f, 0.f};
        accr[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 lo[4], hi[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 x = *(const u32x4*)(ring + qk_off + 64 * (2 * g + half));
          e4m3x16_to_bf16(x, lo[g], hi[g]);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
          for (int hb = 0; hb < NH2; ++hb)
            acc[hb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[g], qreg[hb][2 * (2 * g + half)], acc[hb][g], 0, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
          for (int hb = 0; hb < NH2; ++hb)
            acc[hb][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[g], qreg[hb][2 * (2 * g + half) + 1], acc[hb][g], 0, 0, 0);
        }
      }
      if constexpr (kRope) {
        const bf16x8 r0 = *(const bf16x8*)(ring + (16 * w + li) * RS + 528 + 32 * G);
        const bf16x8 r1 = *(const bf16x8*)(ring + (16 * w + li) * RS + 528 + 32 * G + 16);
#pragma unroll
        for (int hb = 0; hb < NH2; ++hb) {
          accr[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0, qrope[hb][0], accr[hb], 0, 0, 0);
          accr[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r1, qrope[hb][1], accr[hb], 0, 0, 0);
        }
      }
      // fold the rows' scales, mask, write the scores
      f32x4 sc[4];
      if (slot_scaled) {
        const f32x4 ss = *(const f32x4*)&sm.sscale[b][16 * w + 4 * G];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = f32x4{ss[r], ss[r], ss[r], ss[r]};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = *(const f32x4*)(ring + sc_off + r * RS);
      }
#pragma unroll
      for (int hb = 0; hb < NH2; ++hb) {
        f32x4 s;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = accr[hb][r];
#pragma unroll
          for (int g = 0; g < 4; ++g) v += acc[hb][g][r] * sc[r][g];
          s[r] = ((vmw >> (4 * G + r)) & 1u) ? v * p.scale_log2 : kNegInf;
        }
        sm.sx[w][hb][lane] = s;
      }
      // the scale of this wave's dim group for every row (PV)
      if (!slot_scaled) sm.vs[w][lane] = *(const float*)(ring + vs_off);
    }
    barrier_lds();  // scores of all rows visible

    // Q of the next tile's token (the registers are free until its QK^T)
    if (!it1.end && it1.t != it0.t) load_q(it1.t);

    if (any) {
      // ---- online softmax; lane (head li, G) holds rows 32 kk + 8 G + e, e = 0..7
      float pv[NH2][2][8];
#pragma unroll
      for (int hb = 0; hb < NH2; ++hb) {
        float z[2][8];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int wv = 2 * kk + (G >> 1);
          const f32x4 a = sm.sx[wv][hb][16 * (2 * (G & 1)) + li];
          const f32x4 c = sm.sx[wv][hb][16 * (2 * (G & 1) + 1) + li];
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
        const bool bump = tmax > m[hb] + 8.0f;
        const float m_new = bump ? tmax : m[hb];
        const float alpha = bump ? fast_exp2(m[hb] - m_new) : 1.0f;
        float ps = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[hb][kk][e] = (m_new == kNegInf) ? 0.f : fast_exp2(z[kk][e] - m_new);
            ps += pv[hb][kk][e];
          }
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

      // ---- P' = p x scale (this wave's dim group), split into bf16 terms
      float vsc[2][8];
      {
        const float* vsrc = slot_scaled ? sm.sscale[b] : sm.vs[w];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const f32x4 a = *(const f32x4*)(vsrc + 32 * kk + 8 * G);
          const f32x4 c = *(const f32x4*)(vsrc + 32 * kk + 8 * G + 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            vsc[kk][r] = a[r];
            vsc[kk][4 + r] = c[r];
          }
        }
      }
      bf16x8 A[NH2][2][NTERM];
#pragma unroll
      for (int hb = 0; hb < NH2; ++hb) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          float pg[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pg[e] = pv[hb][kk][e] * vsc[kk][e];
          split_terms<NTERM>(pg, A[hb][kk]);
        }
      }

      // ---- O += P' V over dims 128w .. 128w+127, in two halves of 4 dim blocks
      const uint32_t vaddr = lds_u32(ring) + pv_off;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        i32x2 x[4][2];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) x[d][kk] = lds_tr8(vaddr + 32 * kk * RS + 16 * (4 * half + d));
        }
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[1][0]), "+v"(x[1][1]), "+v"(x[2][0]), "+v"(x[2][1]),
                       "+v"(x[3][0]), "+v"(x[3][1]));
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 B = e4m3x8_to_bf16(x[d][kk]);
#pragma unroll
            for (int hb = 0; hb < NH2; ++hb) {
#pragma unroll
              for (int t = 0; t < NTERM; ++t)
                O[hb][4 * half + d] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[hb][kk][t], B, O[hb][4 * half + d], 0, 0, 0);
            }
          }
        }
      }
    }

    if (it1.end || it1.t != it0.t) {
      ep_t = it0.t;
      ep_s = it0.s_first;
      ep_n = it0.nsplit;
    }
    if (it1.end) break;
    it0 = it1;
    it1 = it2;
    it2 = gen_next<kTileRows>(gen, p);
    ++k;
  }
  if (ep_t >= 0) epilogue(ep_t, ep_s, ep_n);
}

template <int DQK, int NH2>
static hipError_t launch_ring_t(const DecodeParams& p, int num_parts, int precision, hipStream_t stream) {
  dim3 grid(num_parts, p.H / (16 * NH2));
  if (precision == 1)
    hipLaunchKernelGGL((decode_ring_kernel<DQK, NH2, 1>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_ring_kernel<DQK, NH2, 3>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_ring(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                              hipStream_t stream) {
  if (d_qk == 576)
    return heads_per_group == 16 ? launch_ring_t<576, 1>(p, num_parts, precision, stream)
                                 : launch_ring_t<576, 2>(p, num_parts, precision, stream);
  return heads_per_group == 16 ? launch_ring_t<512, 1>(p, num_parts, precision, stream)
                               : launch_ring_t<512, 2>(p, num_parts, precision, stream);
}

}  // namespace sda
