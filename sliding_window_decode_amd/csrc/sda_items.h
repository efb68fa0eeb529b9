// sda_items.h -- walks the (token, tile) items of one scheduler part on the device.
//
// A part is the contiguous range [(bt, bi), (et, ei)) of the concatenated per-token tile sequence
// (FlashMLA sparse_decode.h, DecodeImplMeta: begin/end request and block index). Token t's tiles are
// first the ceil(n_main/64) tiles of its main list, then those of its extra list; a token with no
// rows still has one (empty) tile so that its output is written. A kernel may walk each 64-row tile
// as SUB-row items (SUB = 32: two halves, the second only when it holds rows).
//
// The part's first token comes with its lengths and split index in the meta record, so that walking
// starts without a memory round trip. The lengths and split index of each later token are fetched
// when the walker enters the token before it, so that they have long arrived when they are used.
#pragma once

#include "sda_device.h"
#include "sda_internal.h"

namespace sda {

// One item, as wave-uniform scalars: token (-1 past the part's end), list, first list position, list
// length, the token's first split index, and whether this part holds all of the token's tiles (its
// output is then final; otherwise it is one split of the token, number s_first + begin_split for the
// part's first token and s_first for any other).
struct Item {
  int t, L, pos0, n, s_first, whole;
  __device__ __forceinline__ bool end() const { return t < 0; }
};

// Raw lengths of both lists (or their widths) and num_splits[t] of a token.
struct TokenInfo {
  int r0, r1, s0;
};

__device__ __forceinline__ int opaque_lane_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Token information in registers. The load index carries an opaque zero so that the compiler keeps
// the raw values in vector registers (moving them to scalar registers needs the loads complete)
// until the walker enters the token.
struct TokenInfoRegs {
  TokenInfo x;
  __device__ __forceinline__ void issue(const DecodeParams& p, int t) {
    const int tz = t + opaque_lane_zero();
    x.r0 = p.lst[0].lens ? p.lst[0].lens[tz / p.lst[0].lens_div] : p.lst[0].width;
    x.r1 = p.nlists > 1 ? (p.lst[1].lens ? p.lst[1].lens[tz / p.lst[1].lens_div] : p.lst[1].width) : 0;
    x.s0 = p.num_splits[tz];
  }
  __device__ __forceinline__ TokenInfo fetch(const DecodeParams&) const { return x; }
};

struct ItemGen {
  int t, i, j, n0, n1, tm, i_end, t_last, bt, bi, et, ei, s0;
  bool done;
};

__device__ __forceinline__ int clamp_raw(int n, int width) { return n < 0 ? 0 : (n > width ? width : n); }

template <class Src>
__device__ __forceinline__ void gen_enter(ItemGen& g, const DecodeParams& p, Src& src, int t, int r0, int r1, int s0) {
  g.t = t;
  g.n0 = clamp_raw(r0, p.lst[0].width);
  g.n1 = p.nlists > 1 ? clamp_raw(r1, p.lst[1].width) : 0;
  g.s0 = s0;
  g.tm = (g.n0 + kTileRows - 1) / kTileRows;
  g.i = (t == g.bt) ? g.bi : 0;
  g.j = 0;
  g.i_end = (t == g.et) ? g.ei : token_tiles(g.n0, g.n1);
  if (t + 1 <= g.t_last && t + 1 < p.T) src.issue(p, t + 1);
}

// Reads one field in each 64-byte line of the kernel arguments, all in one round trip, so that the
// prologue's later reads of arguments (each issued only behind the branch that needs it) hit the scalar
// cache instead of missing line after line.
__device__ __forceinline__ void touch_args(const DecodeParams& p) {
  static_assert(sizeof(DecodeParams) <= 5 * 64, "one touched field per 64-byte line");
  const uint64_t a = (uint64_t)p.q ^ (uint64_t)p.l_st ^ (uint64_t)p.lst[0].base ^ (uint64_t)p.lst[1].lens;
  const uint32_t b = (uint32_t)p.nlists ^ (uint32_t)p.all_partial;
  asm volatile("" ::"s"(a), "s"(b));
}

// The part record of this workgroup (the layout gen_init reads): row blockIdx.x of the scheduler's meta
// array, or, for a whole-token call (no meta array), token blockIdx.x from its first tile to its end,
// with its clamped lengths read here (one dependent load, in place of the meta record's) and split
// index blockIdx.x (used only when the token leaves as a partial).
__device__ __forceinline__ void part_record(const DecodeParams& p, int32_t (&m)[SDA_META_INTS]) {
  const int b = blockIdx.x;
  if (p.meta) {
    const int32_t* mt = p.meta + (int64_t)b * SDA_META_INTS;
#pragma unroll
    for (int i = 0; i < SDA_META_INTS; ++i) m[i] = mt[i];
    return;
  }
  m[0] = b;
  m[1] = 0;
  m[2] = b + 1;
  m[3] = 0;
  m[4] = 0;
  // scalar loads (through the constant address space): the caller's lengths are not written while
  // the kernel runs
  auto len_of = [&](const ListDev& l) -> int {
    const int n = l.lens ? *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)(l.lens + b / l.lens_div)
                         : l.width;
    return n < 0 ? 0 : (n > l.width ? l.width : n);
  };
  m[5] = b < p.T ? len_of(p.lst[0]) : 0;
  m[6] = (b < p.T && p.nlists > 1) ? len_of(p.lst[1]) : 0;
  m[7] = b;
}

// Starts at the part of meta record m (begin token, begin tile, end token, end tile, begin split,
// clamped main and extra lengths of the begin token, num_splits[begin token]).
template <class Src>
__device__ __forceinline__ void gen_init(ItemGen& g, const DecodeParams& p, Src& src, const int32_t* m) {
  g.bt = m[0];
  g.bi = m[1];
  g.et = m[2];
  g.ei = m[3];
  g.t_last = (g.ei > 0) ? g.et : g.et - 1;
  g.done = false;
  gen_enter(g, p, src, g.bt, m[5], m[6], m[7]);
}

// Next item; list L's items have sub[L] rows (64, or 32: tile halves, the second only when it holds
// rows).
// before_fetch() runs just before the walker reads a token's fetched information.
template <class Src, class Wait>
__device__ __forceinline__ Item gen_next_sub(ItemGen& g, const DecodeParams& p, Src& src, int sub0, int sub1,
                                             Wait&& before_fetch) {
  Item it;
  if (g.done) {
    it.t = -1;
    it.L = 0;
    it.pos0 = 0;
    it.n = 0;
    it.s_first = 0;
    it.whole = 1;
    return it;
  }
  it.t = g.t;
  it.s_first = g.s0;
  it.whole = (g.t != g.bt || g.bi == 0) && (g.t != g.et || g.ei == 0);
  it.L = g.i < g.tm ? 0 : 1;
  it.n = it.L == 0 ? g.n0 : g.n1;
  const int sub = it.L == 0 ? sub0 : sub1;
  it.pos0 = kTileRows * (it.L == 0 ? g.i : g.i - g.tm) + sub * g.j;
  if (sub < kTileRows && g.j + 1 < kTileRows / sub && it.pos0 + sub < it.n) {
    g.j += 1;
  } else if (g.i + 1 < g.i_end) {
    g.i += 1;
    g.j = 0;
  } else if (g.t + 1 <= g.t_last && g.t + 1 < p.T) {
    before_fetch();
    const TokenInfo x = src.fetch(p);
    gen_enter(g, p, src, g.t + 1, __builtin_amdgcn_readfirstlane(x.r0), __builtin_amdgcn_readfirstlane(x.r1),
              __builtin_amdgcn_readfirstlane(x.s0));
  } else {
    g.done = true;
  }
  return it;
}

template <int SUB, class Src>
__device__ __forceinline__ Item gen_next(ItemGen& g, const DecodeParams& p, Src& src) {
  return gen_next_sub(g, p, src, SUB, SUB, [] {});
}

template <int SUB, class Src, class Wait>
__device__ __forceinline__ Item gen_next(ItemGen& g, const DecodeParams& p, Src& src, Wait&& before_fetch) {
  return gen_next_sub(g, p, src, SUB, SUB, before_fetch);
}

}  // namespace sda
