// sda_items.h -- walks the (token, tile) items of one scheduler part on the device.
//
// A part is the contiguous range [(bt, bi), (et, ei)) of the concatenated per-token tile sequence
// (FlashMLA sparse_decode.h, DecodeImplMeta: begin/end request and block index). Token t's tiles are
// first the ceil(n_main/64) tiles of its main list, then those of its extra list; a token with no
// rows still has one (empty) tile so that its output is written. A kernel may walk each 64-row tile
// as SUB-row items (SUB = 32: two halves, the second only when it holds rows).
#pragma once

#include "sda_internal.h"

namespace sda {

// One item, as wave-uniform scalars: token, list, first list position, list length, end marker, and
// the token's split range (first split index, number of splits).
struct Item {
  int t, L, pos0, n, end, s_first, nsplit;
};

// The lengths and split range of the next token are loaded when the walker enters a token, so that
// the loads are long complete when they are used (a load consumed right away would make the wave
// wait for every global load in flight, the gathers included). The raw values stay in vector
// registers until then: the load index carries an opaque zero so that the compiler does not move
// them to scalar registers (which needs the load to be complete) straight after the load.
struct TokenInfo {
  int r0, r1, s0, s1;  // raw lens of both lists (or their widths), num_splits[t], num_splits[t + 1]
};

__device__ __forceinline__ int opaque_lane_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

struct ItemGen {
  int t, i, j, n0, n1, tm, i_end, t_last, bt, bi, et, ei, s0, s1;
  TokenInfo next;
  bool done;
};

__device__ __forceinline__ TokenInfo load_token_info(const DecodeParams& p, int t) {
  const int tz = t + opaque_lane_zero();
  TokenInfo x;
  x.r0 = p.lst[0].lens ? p.lst[0].lens[tz] : p.lst[0].width;
  x.r1 = p.nlists > 1 ? (p.lst[1].lens ? p.lst[1].lens[tz] : p.lst[1].width) : 0;
  x.s0 = p.num_splits[tz];
  x.s1 = p.num_splits[tz + 1];
  return x;
}

__device__ __forceinline__ int clamp_raw(int n, int width) { return n < 0 ? 0 : (n > width ? width : n); }

__device__ __forceinline__ void gen_enter(ItemGen& g, const DecodeParams& p, int t, const TokenInfo& x) {
  g.t = t;
  g.n0 = clamp_raw(__builtin_amdgcn_readfirstlane(x.r0), p.lst[0].width);
  g.n1 = p.nlists > 1 ? clamp_raw(__builtin_amdgcn_readfirstlane(x.r1), p.lst[1].width) : 0;
  g.s0 = __builtin_amdgcn_readfirstlane(x.s0);
  g.s1 = __builtin_amdgcn_readfirstlane(x.s1);
  g.tm = (g.n0 + kTileRows - 1) / kTileRows;
  g.i = (t == g.bt) ? g.bi : 0;
  g.j = 0;
  g.i_end = (t == g.et) ? g.ei : token_tiles(g.n0, g.n1);
  if (t + 1 <= g.t_last && t + 1 < p.T) g.next = load_token_info(p, t + 1);
}

__device__ __forceinline__ void gen_init(ItemGen& g, const DecodeParams& p, int bt, int bi, int et, int ei) {
  g.bt = bt;
  g.bi = bi;
  g.et = et;
  g.ei = ei;
  g.t_last = (ei > 0) ? et : et - 1;
  g.done = false;
  gen_enter(g, p, bt, load_token_info(p, bt));
}

// Next item; list L's items have sub[L] rows (64, or 32: tile halves, the second only when it holds
// rows).
__device__ __forceinline__ Item gen_next_sub(ItemGen& g, const DecodeParams& p, int sub0, int sub1) {
  Item it;
  if (g.done) {
    it.t = -1;
    it.L = 0;
    it.pos0 = 0;
    it.n = 0;
    it.end = 1;
    it.s_first = 0;
    it.nsplit = 0;
    return it;
  }
  it.t = g.t;
  it.s_first = g.s0;
  it.nsplit = g.s1 - g.s0;
  it.L = g.i < g.tm ? 0 : 1;
  it.n = it.L == 0 ? g.n0 : g.n1;
  const int sub = it.L == 0 ? sub0 : sub1;
  it.pos0 = kTileRows * (it.L == 0 ? g.i : g.i - g.tm) + sub * g.j;
  it.end = 0;
  if (sub < kTileRows && g.j + 1 < kTileRows / sub && it.pos0 + sub < it.n) {
    g.j += 1;
  } else if (g.i + 1 < g.i_end) {
    g.i += 1;
    g.j = 0;
  } else if (g.t + 1 <= g.t_last && g.t + 1 < p.T) {
    gen_enter(g, p, g.t + 1, g.next);
  } else {
    g.done = true;
  }
  return it;
}

template <int SUB>
__device__ __forceinline__ Item gen_next(ItemGen& g, const DecodeParams& p) {
  return gen_next_sub(g, p, SUB, SUB);
}

}  // namespace sda
