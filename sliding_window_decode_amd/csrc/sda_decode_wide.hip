// sda_decode_wide.hip -- decode attention over 576-dim records (SDA_V32_656: 512 fp8 dims with one fp32
// scale per 128 dims, then 64 bf16 dims) for 64 query heads per workgroup, on gfx950.
//
// Workgroup = one scheduler part (or one token, for a whole-token plan) x 64 heads; eight waves, two per
// SIMD, so that one wave's conversions, softmax and gather issue run while the other's matrix products do.
// Every product is a v_mfma_f32_32x32x16_bf16: one widened 32 x 16 operand fragment feeds 32 heads (the
// 16x16x32 product feeds 16), which halves the fp8 widening per head. Per tile k:
//   gather  tile k+1's records into the other of two LDS ring buffers (global -> LDS, 16 bytes a lane,
//           656-byte rows: an odd number of 16-byte chunks), each record's four fp32 scales into a per-row
//           table and 0 or -inf into a per-row mask; masked rows (slot -1, out of range, past the length)
//           read a zero record. Waves 0 .. 3 turn the slot ids into addresses at the top of the tile and
//           issue the loads once the softmax is done, waiting on the address unit while waves 4 .. 7 run PV
//   QK^T    wave (hb, dh, rb): heads 32 hb .. 32 hb + 31, rows 32 rb .. 32 rb + 31, dims half dh (fp8 dims
//           256 dh .. +255, rope dims 512 + 32 dh .. +31): S^T = K Q^T with rows on M and heads on N; K's
//           fp8 codes are widened (exactly) as read, one accumulator per 128-dim scale group folded with
//           the rows' scales after its products; the partial scores go to LDS
//   softmax wave w: heads 8 w .. 8 w + 7, the eight lanes of a head holding its 64 rows (the two dims
//           halves' partial scores summed, masked rows at -inf); online softmax in base 2 (the reference
//           max moves only when a tile exceeds it by more than 8), reductions by DPP within the eight
//           lanes; the weights p go to LDS in the PV operand layout, each head's rescale factor beside them
//   PV      wave (hb, g): output dims 128 g .. 128 g + 127 (scale group g) of heads 32 hb .. 32 hb + 31:
//           O^T += V^T P'^T with P' = p x the rows' scale of group g split into NTERM bf16 terms, V read
//           transposed from the fp8 ring rows with ds_read_b64_tr_b8 and widened
// A token's output leaves after its last tile in the part: the final bf16 row and LSE (sink folded in)
// when the part holds the whole token, else a normalized fp32 partial and its LSE for the combine.
//
// Sources: masked softmax attention (native_swa_decode.py, _fallback_batched_sdp); gather, validity
// and page addressing (vLLM swapab_decode_attn, stage_inputs); online softmax (native_swa_decode.py,
// BlackwellSWADecodeKernel); swap-AB score product, P = hi + lo and the sink merge (vLLM
// swapab_decode_attn, device kernel steps 3, 4 and 9); split buffers (FlashMLA sparse_decode.h,
// o_accum / lse_accum); the 656-byte record (FlashMLA sparse_decode.h, V3.2 bytes_per_token).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sda_device.h"
#include "sda_internal.h"
#include "sda_items.h"

namespace sda {

namespace {

// Masked rows gather from here: zero codes, zero scales and zero rope dims.
__device__ __attribute__((aligned(16))) uint8_t g_zero_record_wide[1024];

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kRec = 656;                           // record bytes (41 chunks of 16 bytes)
constexpr int kNC = kRec / 16;                      // chunks per record
constexpr int kNB = 2;                              // ring buffers
constexpr int kGW = 4;                              // gathering waves (0 .. 3)
constexpr int kNI = (kNC + kGW - 1) / kGW;          // gather instructions per gathering wave and tile (11)
constexpr int kPP = 20;                             // floats per (head, k-step) row of the weights array
constexpr int kCS = 1088;                           // ring bytes per chunk of all 64 rows (1024 + 64)

// The LDS serves a 16-byte access of 16 lanes, or an 8-byte access of 32, per cycle (256 bytes over 64
// 4-byte banks); lanes in the same bank at different addresses take turns. The layouts below are padded
// or swizzled so that every access of the kernel hits distinct banks.
//
// Ring buffers are chunk-major: chunk q (bytes 16 q .. 16 q + 15 of the record) of row r sits at byte
// 1088 q + 16 r. One global -> LDS load then moves chunk q of all 64 rows (lane r: row r, lane-contiguous
// destinations), its source the lane's record address plus a constant. (The 64 bytes after each chunk's
// 1024 put the two chunks that a transposed V read takes at different banks.)
__device__ __forceinline__ uint32_t ring_off(int q, int r) { return (uint32_t)(kCS * q + 16 * r); }

// Partial scores are written lane-contiguously and read by the softmax lanes 32 rows apart: entry
// (row block rb, 4-row group a, lane l) sits at lane slot l ^ 2 sx_swz(rb, a, l), so that the 16 lanes of
// a softmax read, which take 8 (rb, a / 2, l / 32) combinations, hit 16 distinct slots.
__device__ __forceinline__ int sx_slot(int rb, int a, int l) {
  return l ^ ((((rb & 1) << 2) | (((a >> 1) & 1) << 1) | ((l >> 5) & 1)) << 1);
}

// softmax weights of one (head block, k-step): [head][8 hf + e] (16 of kPP used), then 16 floats that
// offset the next k-step's block by 64 bytes modulo 256 (the softmax lanes store four k-steps at once)
struct PwBlock {
  float v[32][kPP];
  float pad[16];
};

struct WideSmem {
  char ring[kNB][kNC * kCS];
  // partial scores: [dims half][head block][row block][4-row group a][lane slot] in the 32x32 accumulator
  // layout (sx_slot)
  f32x4 sx[2][2][2][4][64];
  // softmax weights in the PV operand layout: [head block][k-step]
  __attribute__((aligned(16))) PwBlock pw[2][4];
  // each row's four fp32 scales: [buffer][scale group][row]
  __attribute__((aligned(16))) float stab[kNB][4][kTileRows];
  // each row's additive score mask: 0 for a valid row, -inf for a masked one
  __attribute__((aligned(16))) float mtab[kNB][kTileRows];
  float alpha[64];      // per head: factor the running output is rescaled by in this tile
  float hinv[64];       // per head: factor the token's output is multiplied by in its epilogue
  uint32_t vany[kNB];  // whether the tile has a valid row
};

// DPP lane exchanges within groups of eight consecutive lanes (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max_of_8(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  return fmaxf(v, dpp_f<0x141>(v));
}
__device__ __forceinline__ float sum_of_8(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  return v + dpp_f<0x141>(v);
}

// fp32 values split into NTERM bf16 terms whose sum reproduces them (exactly for NTERM = 3), converting two
// values per instruction (v_cvt_pk_bf16_f32, round to nearest even)
template <int NTERM>
__device__ __forceinline__ void split_pairs(const float (&v)[8], bf16x8 (&A)[NTERM]) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = v[e];
#pragma unroll
  for (int k = 0; k < NTERM; ++k) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 h = bf16x2{(__bf16)r[e], (__bf16)r[e + 1]};
      A[k][e] = h[0];
      A[k][e + 1] = h[1];
      if (k + 1 < NTERM) {
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        r[e] -= __builtin_bit_cast(float, hb << 16);
        r[e + 1] -= __builtin_bit_cast(float, hb & 0xFFFF0000u);
      }
    }
  }
}

}  // namespace

// NTERM: bf16 terms of P' in the P.V product (1, 2 or 3).
template <int NTERM>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_wide_kernel(DecodeParams p) {
  __shared__ WideSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;                         // 32x32 operand layout: column / row, k half
  const int qhb = w >> 2, qdh = (w >> 1) & 1, qrb = w & 1;         // QK^T: head block, dims half, row block
  const int h8 = lane >> 3, sq = lane & 7;                         // softmax: head 8 w + h8, its eighth sq
  const int srb = sq >> 2, shf = (sq >> 1) & 1, sah = sq & 1;      // rows 32 srb + 8 (2 sah + a0) + 4 shf + e
  const int phb = w >> 2, pg = w & 3;                              // PV: head block, scale group
  const int h0 = blockIdx.y * 64;

  auto LD = [&](int L) -> const ListDev& { return p.lst[L]; };
  touch_args(p);
  // A whole-token call knows its token before its lengths arrive: the slot ids of list 0's first two tiles
  // are loaded first (positions clamped below the width: always readable) and kept for the first items
  // that turn out to be those tiles.
  const bool spec = p.meta == nullptr;
  int sid_spec[kNB];
  {
    const ListDev& l0 = LD(0);
    const int tb = blockIdx.x < (unsigned)p.T ? (int)blockIdx.x : 0;
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      const int pos = kTileRows * j + lane;
      sid_spec[j] = l0.idx[(int64_t)tb * l0.row_stride + (pos < l0.width ? pos : l0.width - 1)];
    }
  }
  asm volatile("" ::: "memory");
  int32_t mrec[SDA_META_INTS];
  part_record(p, mrec);
  const int bt = mrec[0], bi = mrec[1], et = mrec[2], ei = mrec[3], bk = mrec[4];
  if (bt >= p.T || bt > et || (bt == et && bi >= ei)) return;

  // softmax lanes: head 8 w + h8's sink logit in log2 units
  const float sink2 = p.sink ? p.sink[h0 + 8 * w + h8] * kLog2e : kNegInf;

  auto load_sid = [&](const Item& it) -> int {
    int sid = -1;
    if (!it.end()) {
      const int pos = it.pos0 + lane;  // lane: row of the tile
      const ListDev& ld = LD(it.L);
      if (pos < it.n) sid = ld.idx[(int64_t)it.t * ld.row_stride + pos];
    }
    return sid;
  };
  const uint64_t zero_rec = (uint64_t)(const void*)g_zero_record_wide;
  // The gather of a tile's records is issued by waves 0 .. 3 alone, each taking every fourth chunk of all 64
  // rows: the address unit takes the loads in turn, and while those waves wait to issue, waves 4 .. 7 (which
  // share their SIMDs) run their PV products. gather_rows turns the lane's slot id (row `lane` of the tile)
  // into its record address (a masked row: the zero record) and, in wave 0, writes the rows' score masks and
  // whether any row is valid; gather_issue then issues this wave's loads into ring buffer b: chunks
  // w + 4 i of every row (source: the row's address plus a constant offset) and scale group w of every row.
  auto gather_rows = [&](const Item& it, int sid, int b) -> uint64_t {
    const ListDev& ld = LD(it.L);
    const bool ok = sid >= 0 && sid < ld.slots;
    uint64_t ra = zero_rec;
    if (ok) {
      const uint32_t pg_ = (uint32_t)sid >> ld.page_shift;
      const uint32_t off = (uint32_t)sid & ((1u << ld.page_shift) - 1u);
      ra = (uint64_t)ld.base + (uint64_t)pg_ * (uint64_t)ld.page_stride + (uint64_t)off * (uint64_t)kRec;
    }
    if (w == 0) {
      sm.mtab[b][lane] = ok ? 0.0f : kNegInf;
      const uint64_t vm = __ballot(ok);
      if (lane == 0) sm.vany[b] = vm != 0 ? 1u : 0u;
    }
    return ra;
  };
  auto gather_issue_part = [&](uint64_t ra, int b, auto i0c, auto i1c) {
    constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
    const uint64_t src = ra + 16 * w;
    char* dst = sm.ring[b] + kCS * w;
    // load i moves chunk w + kGW i: source byte 16 (w + kGW i) of the record, the kGW i part carried in the
    // load's immediate, which the hardware adds to the LDS destination too (the base given is that much
    // below chunk w + kGW i); chunks past the record's last (w + kGW i >= kNC) are not loaded
    static_assert(16 * kGW * (kNI - 1) < 4096, "offsets fit the load's immediate");
    static_assert(kGW == 4, "the four gathering waves load one scale group each");
    static_for<I0, I1>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (w + kGW * i < kNC) dma16_at<16 * kGW * i>(src, dst + (kCS - 16) * kGW * i);
    });
    if constexpr (I1 == kNI) dma4(ra + 512 + 4 * w, &sm.stab[b][w][0]);
  };
  auto gather_issue = [&](uint64_t ra, int b) {
    gather_issue_part(ra, b, std::integral_constant<int, 0>{}, std::integral_constant<int, kNI>{});
  };

  // ---- prologue: items k = 0 .. 2, the gather of tile 0 in flight, the slot ids of tile 1
  ItemGen gen;
  TokenInfoRegs tinfo;
  gen_init(gen, p, tinfo, mrec);
  Item its[kNB + 1];  // its[j] = tile k + j
#pragma unroll
  for (int j = 0; j <= kNB; ++j) its[j] = gen_next<kTileRows>(gen, p, tinfo);
  int sid_next = -1;
  if (w < kGW) {
    int sids[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      if (spec && !its[j].end() && its[j].L == 0 && its[j].pos0 == kTileRows * j)
        sids[j] = kTileRows * j + lane < its[j].n ? sid_spec[j] : -1;
      else
        sids[j] = load_sid(its[j]);
    }
    gather_issue(gather_rows(its[0], sids[0], 0), 0);
    sid_next = sids[1];
  }

  // Q of this wave's QK^T role: head h0 + 32 qhb + n, k-step (scale group 2 qdh + gi, pair s2, j): dims
  // 128 (2 qdh + gi) + 32 s2 + 16 hf + 8 j + 0..7; rope k-step r: dims 512 + 32 qdh + 16 r + 8 hf + 0..7
  bf16x8 qf[2][4][2];
  bf16x8 qr[2];
  auto load_q = [&](int t) {
    const uint16_t* qh = p.q + (int64_t)t * p.q_st + (int64_t)(h0 + 32 * qhb + n) * p.q_sh;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const uint16_t* src = qh + 128 * (2 * qdh + gi) + 32 * s2 + 16 * hf;
        qf[gi][s2][0] = *(const bf16x8*)src;
        qf[gi][s2][1] = *(const bf16x8*)(src + 8);
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) qr[r] = *(const bf16x8*)(qh + 512 + 32 * qdh + 16 * r + 8 * hf);
  };
  load_q(its[0].t);

  // PV state: O^T blocks [dim block db of this wave's 128 dims], 32x32 accumulator layout (lane: head
  // 32 phb + n, dims 128 pg + 32 db + 8 (r / 4) + 4 hf + r % 4)
  f32x16 O[4];
  auto reset_o = [&]() {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) O[db][r] = 0.f;
    }
  };
  reset_o();
  // softmax state of head 8 w + h8 (the running max is the same in the head's eight lanes; l is the sum
  // over this lane's rows)
  float m = kNegInf, l = 0.f;

  int k = 0;
  while (true) {
    const int b = k & 1;
    vm_wait<0>();   // tile k's gather (issued one iteration earlier) and everything before it landed
    barrier_lds();  // every wave's gather of tile k landed; ring buffer b ^ 1 is free

    // slot ids of tile k+2, then the gather of tile k+1 into the free buffer (its loads issued below)
    const bool gwave = w < kGW;
    const int sid_new = gwave ? load_sid(its[2]) : -1;
    const bool gath = gwave && !its[1].end();
    uint64_t ra_next = 0;
    if (gath) ra_next = gather_rows(its[1], sid_next, b ^ 1);
    sid_next = sid_new;

    const Item it0 = its[0], it1 = its[1];
    const bool last = it1.end() || it1.t != it0.t;  // tile k is the token's last in this part
    const char* ring = sm.ring[b];
    const uint32_t vany = sm.vany[b];

    // ---- QK^T: partial scores of this wave's head block, row block and dims half
    if (vany) {
      const int qrow = 32 * qrb + n;  // the lane's row
      f32x16 S;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = 0.f;
      // rope dims: bf16 as stored (no scale)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(ring + ring_off(33 + 4 * qdh + hf + 2 * r, qrow)),
                                                    qr[r], S, 0, 0, 0);
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int g = 2 * qdh + gi;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const u32x4 x = *(const u32x4*)(ring + ring_off(8 * g + 2 * s2 + hf, qrow));
          bf16x8 lo, hi;
          e4m3x16_to_bf16_scaled(x, 1.0f, lo, hi);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, qf[gi][s2][0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, qf[gi][s2][1], acc, 0, 0, 0);
        }
        // fold the rows' scales of group g: lane rows 32 qrb + 8 a + 4 hf + 0..3
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 sc = *(const f32x4*)&sm.stab[b][g][32 * qrb + 8 * a + 4 * hf];
#pragma unroll
          for (int e = 0; e < 4; ++e) S[4 * a + e] = __builtin_fmaf(acc[4 * a + e], sc[e], S[4 * a + e]);
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
        sm.sx[qdh][qhb][qrb][a][sx_slot(qrb, a, lane)] = f32x4{S[4 * a], S[4 * a + 1], S[4 * a + 2], S[4 * a + 3]};
    }
    barrier_lds();  // partial scores visible
    // the first three of the gather loads of tile k+1 (the rest follow the softmax, below)
    if (gath) gather_issue_part(ra_next, b ^ 1, std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});

    // Q of the next tile's token (the registers are free until its QK^T)
    if (!it1.end() && it1.t != it0.t) load_q(it1.t);

    // ---- online softmax of heads 8 w .. 8 w + 7: lane (h8, sq) holds rows 32 srb + 8 (2 sah + a0) + 4 shf + e
    if (vany) {
      const int src_lane = 8 * (w & 3) + h8 + 32 * shf;
      float z[2][4];
#pragma unroll
      for (int a0 = 0; a0 < 2; ++a0) {
        const int a = 2 * sah + a0;
        const f32x4 x0 = sm.sx[0][w >> 2][srb][a][sx_slot(srb, a, src_lane)];
        const f32x4 x1 = sm.sx[1][w >> 2][srb][a][sx_slot(srb, a, src_lane)];
        const f32x4 mk = *(const f32x4*)&sm.mtab[b][32 * srb + 8 * a + 4 * shf];
#pragma unroll
        for (int e = 0; e < 4; ++e) z[a0][e] = __builtin_fmaf(x0[e] + x1[e], p.scale_log2, mk[e]);
      }
      float tmax = fmaxf(fmaxf(fmaxf(z[0][0], z[0][1]), fmaxf(z[0][2], z[0][3])),
                         fmaxf(fmaxf(z[1][0], z[1][1]), fmaxf(z[1][2], z[1][3])));
      tmax = max_of_8(tmax);
      const bool bump = tmax > m + 8.0f;
      const float m_new = bump ? tmax : m;
      const float alpha = bump ? fast_exp2(m - m_new) : 1.0f;
      const float mref = m_new == kNegInf ? 0.f : m_new;  // all rows masked so far: exp2(-inf) = 0
      float ps = 0.f;
      f32x4 pv[2];
#pragma unroll
      for (int a0 = 0; a0 < 2; ++a0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[a0][e] = fast_exp2(z[a0][e] - mref);
          ps += pv[a0][e];
        }
      }
      // PV operand layout: k-step 2 srb + sah, row half shf, elements 4 a0 + e
      float* pdst = &sm.pw[w >> 2][2 * srb + sah].v[8 * (w & 3) + h8][8 * shf];
      *(f32x4*)pdst = pv[0];
      *(f32x4*)(pdst + 4) = pv[1];
      l = l * alpha + ps;
      m = m_new;
      if (sq == 0) sm.alpha[8 * w + h8] = alpha;
    } else if (sq == 0) {
      sm.alpha[8 * w + h8] = 1.0f;
    }
    if (last) {
      // the token's output factor and LSE (sink folded in when the part holds the whole token)
      const bool whole = it0.whole && !p.all_partial;
      const float lt = sum_of_8(l);
      float inv, lse_out;
      token_output_factor(m, lt, sink2, whole, inv, lse_out);
      if (sq == 0) {
        const int h = h0 + 8 * w + h8;
        sm.hinv[8 * w + h8] = inv;
        if (whole)
          p.lse[(int64_t)it0.t * p.l_st + h] = lse_out;
        else
          p.lse_acc[(int64_t)(it0.s_first + (it0.t == bt ? bk : 0)) * p.H + h] = lse_out;
      }
      m = kNegInf;
      l = 0.f;
    }
    barrier_lds();  // weights, rescale factors and output factors visible
    // The rest of the gather loads of tile k+1, issued here rather than with the addresses above: the address
    // unit takes about as long to accept a tile's loads as a SIMD needs for one wave's PV, so waves 0 .. 3
    // wait for it while waves 4 .. 7, which share their SIMDs, run their PV products (issued at the top of
    // the tile they held waves 0 .. 3 past the QK^T that waves 4 .. 7 finish sooner; three of the eleven
    // issued before the softmax let the tile land sooner at little cost to it: 1-2 % faster than none or
    // six).
    if (gath) gather_issue_part(ra_next, b ^ 1, std::integral_constant<int, 3>{}, std::integral_constant<int, kNI>{});

    // ---- PV over dims 128 pg .. 128 pg + 127 of heads 32 phb .. 32 phb + 31
    {
      const float al = sm.alpha[32 * phb + n];
      if (__any(al != 1.0f)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int r = 0; r < 16; ++r) O[db][r] *= al;
        }
      }
    }
    if (vany) {
      // k-step kk covers rows 16 kk .. 16 kk + 15; row half hf holds rows 16 kk + 8 (e / 4) + 4 hf + e % 4
      // (those the softmax lanes wrote): the transposed V reads point lane pair (2e, 2e+1) of each 16-lane
      // group at that row, the group's k half being G / 2
      const int G = lane >> 4, j = lane & 15;
      const int er = j >> 1;
      const uint32_t vrow = (uint32_t)(8 * (er >> 2) + 4 * (G >> 1) + (er & 3));
      // dims 128 pg + 32 db + 16 (G & 1) + 8 (j & 1) + 0..7: chunk 8 pg + 2 db + (G & 1), bytes 8 (j & 1) ..
      const uint32_t vbase = lds_u32(ring) + ring_off(8 * pg + (G & 1), vrow) + 8 * (j & 1);
      static_for<0, 4>([&](auto kc) {
        constexpr int kk = decltype(kc)::value;
        i32x2 x[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) x[db] = lds_tr8(vbase + ring_off(2 * db, 16 * kk));
        // P' = p x the rows' scale of group pg (rows 16 kk + 8 c + 4 hf + 0..3), split into bf16 terms
        bf16x8 A[NTERM];
        {
          const f32x4 s0 = *(const f32x4*)&sm.stab[b][pg][16 * kk + 4 * hf];
          const f32x4 s1 = *(const f32x4*)&sm.stab[b][pg][16 * kk + 8 + 4 * hf];
          const f32x4 p0 = *(const f32x4*)&sm.pw[phb][kk].v[n][8 * hf];
          const f32x4 p1 = *(const f32x4*)&sm.pw[phb][kk].v[n][8 * hf + 4];
          float pg8[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pg8[e] = p0[e] * s0[e];
            pg8[4 + e] = p1[e] * s1[e];
          }
          split_pairs<NTERM>(pg8, A);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 V = e4m3x8_to_bf16(x[db]);
#pragma unroll
          for (int t = 0; t < NTERM; ++t) O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(V, A[t], O[db], 0, 0, 0);
        }
      });
    }


    if (last) {
      // ---- the token's output rows: head h0 + 32 phb + n, dims 128 pg + 32 db + 8 a + 4 hf + 0..3
      const bool whole = it0.whole && !p.all_partial;
      const float iv = sm.hinv[32 * phb + n];
      if (whole) {
        uint16_t* orow = p.out + (int64_t)it0.t * p.o_st + (int64_t)(h0 + 32 * phb + n) * p.o_sh + 128 * pg + 4 * hf;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const uint32_t lo = (uint32_t)f32_to_bf16_bits(O[db][4 * a] * iv) |
                                ((uint32_t)f32_to_bf16_bits(O[db][4 * a + 1] * iv) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_bits(O[db][4 * a + 2] * iv) |
                                ((uint32_t)f32_to_bf16_bits(O[db][4 * a + 3] * iv) << 16);
            *(u32x2*)(orow + 32 * db + 8 * a) = u32x2{lo, hi};
          }
        }
      } else {
        const int s = it0.s_first + (it0.t == bt ? bk : 0);
        float* orow = p.o_acc + ((int64_t)s * p.H + h0 + 32 * phb + n) * kDv + 128 * pg + 4 * hf;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
          for (int a = 0; a < 4; ++a)
            *(f32x4*)(orow + 32 * db + 8 * a) =
                f32x4{O[db][4 * a] * iv, O[db][4 * a + 1] * iv, O[db][4 * a + 2] * iv, O[db][4 * a + 3] * iv};
        }
      }
      reset_o();
    }

    if (it1.end()) break;
#pragma unroll
    for (int jj = 0; jj < kNB; ++jj) its[jj] = its[jj + 1];
    its[kNB] = gen_next<kTileRows>(gen, p, tinfo);
    ++k;
  }
}

// 576-dim records (every list SDA_V32_656), 64 heads per workgroup: eight waves, one workgroup per CU.
hipError_t launch_decode_wide(const DecodeParams& p, int num_parts, int precision, hipStream_t stream) {
  dim3 grid(num_parts, p.H / 64);
  const dim3 block(64 * kWaves);
  if (precision == 1)
    hipLaunchKernelGGL((decode_wide_kernel<1>), grid, block, 0, stream, p);
  else if (precision == 2)
    hipLaunchKernelGGL((decode_wide_kernel<2>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_wide_kernel<3>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace sda
