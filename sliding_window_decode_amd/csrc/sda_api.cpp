// sda_api.cpp -- host side of the C ABI declared in include/sda.h: argument checks, the plan, the
// workspace layout and the kernel launches. Nothing here allocates device memory or synchronizes.
//
// The checks follow the validation block of FlashMLA sparse_decode.h (sparse_attn_decode_interface):
// MQA only (one latent row per slot), d_qk in {576, 512} with d_v = 512, a positive list width,
// the extra cache and extra indices given together, and record sizes that match the format.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "sda_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
  return SDA_ERR_HIP;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int64_t v) {
  int s = 0;
  while ((int64_t(1) << s) < v) ++s;
  return s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool supported_heads(int H) { return H == 16 || H == 32 || H == 64 || H == 128; }

int check_cache(const sda_cache* c, int d_qk, const char* which) {
  static char msg[256];
  if (!c || !c->base) {
    snprintf(msg, sizeof(msg), "%s cache: NULL", which);
    return fail(SDA_ERR_INVALID_ARG, msg);
  }
  const int rec = sda_record_bytes(c->format);
  if (rec < 0) {
    snprintf(msg, sizeof(msg), "%s cache: unknown format %d", which, c->format);
    return fail(SDA_ERR_UNSUPPORTED, msg);
  }
  if (sda_format_dims(c->format) != d_qk) {
    snprintf(msg, sizeof(msg), "%s cache: format %d holds %d dims, d_qk is %d", which, c->format,
             sda_format_dims(c->format), d_qk);
    return fail(SDA_ERR_UNSUPPORTED, msg);
  }
  if (!aligned(c->base, 16)) return fail(SDA_ERR_INVALID_ARG, "cache base must be 16-byte aligned");
  if (c->num_pages < 1 || !is_pow2(c->page_size))
    return fail(SDA_ERR_INVALID_ARG, "cache needs num_pages >= 1 and a power-of-two page_size");
  if (c->num_pages * (int64_t)c->page_size >= (int64_t(1) << 31))
    return fail(SDA_ERR_INVALID_ARG, "cache holds 2^31 slots or more");
  if (c->page_stride < (int64_t)c->page_size * rec || (c->page_stride % 16) != 0)
    return fail(SDA_ERR_INVALID_ARG, "page_stride must be >= page_size * record bytes and a multiple of 16");
  if ((c->format == SDA_FP8_SLOTSCALE) != (c->slot_scale != nullptr))
    return fail(SDA_ERR_INVALID_ARG, "slot_scale is required for SDA_FP8_SLOTSCALE and only for it");
  return SDA_OK;
}

int check_list(const sda_list* l, const char* which) {
  static char msg[256];
  if (!l || !l->idx) {
    snprintf(msg, sizeof(msg), "%s list: NULL", which);
    return fail(SDA_ERR_INVALID_ARG, msg);
  }
  if (l->width < 1 || l->row_stride < l->width) {
    snprintf(msg, sizeof(msg), "%s list: width must be >= 1 and row_stride >= width", which);
    return fail(SDA_ERR_INVALID_ARG, msg);
  }
  if (l->queries_per_len < 0) {
    snprintf(msg, sizeof(msg), "%s list: queries_per_len must be >= 0", which);
    return fail(SDA_ERR_INVALID_ARG, msg);
  }
  return SDA_OK;
}

// Tokens per length entry of a list (0 means one entry per token).
int lens_div(const sda_list* l) { return l->queries_per_len > 1 ? l->queries_per_len : 1; }

int check_plan(const sda_plan* plan, int H) {
  if (!plan) return fail(SDA_ERR_INVALID_ARG, "plan is NULL");
  if (plan->num_parts < 1 || plan->num_parts > (1 << 20)) return fail(SDA_ERR_INVALID_ARG, "plan.num_parts out of range");
  const int hb = plan->heads_per_group;
  if (!(hb == 16 || hb == 32 || hb == 64) || H % hb != 0)
    return fail(SDA_ERR_UNSUPPORTED, "plan.heads_per_group must be 16, 32 or 64 and divide H");
  if (plan->fixed_overhead < 0 || plan->fixed_overhead > 1024)
    return fail(SDA_ERR_INVALID_ARG, "plan.fixed_overhead out of range");
  if (plan->precision < 1 || plan->precision > 3) return fail(SDA_ERR_INVALID_ARG, "plan.precision must be 1, 2 or 3");
  if (plan->whole_tokens != 0 && plan->whole_tokens != 1)
    return fail(SDA_ERR_INVALID_ARG, "plan.whole_tokens must be 0 or 1");
  return SDA_OK;
}

// The schedulers (device and host) and the decode kernels' part walk count tile positions in 32-bit
// integers: T x (the most tiles a token can take + fixed_overhead) must stay below 2^31.
int check_cost_range(int T, int width, int extra_width, const sda_plan* plan) {
  const int64_t per_token = ((int64_t)width + 63) / 64 + ((int64_t)extra_width + 63) / 64 + 1 + plan->fixed_overhead;
  if ((int64_t)T * per_token >= (int64_t(1) << 31))
    return fail(SDA_ERR_UNSUPPORTED, "T x (tiles per token + fixed_overhead) must stay below 2^31");
  return SDA_OK;
}

struct WorkspaceLayout {
  size_t o_acc, lse_acc, meta, num_splits, total;
  size_t q_rot, total_v41;  // V4.1 calls: the rotated q after everything else
};

WorkspaceLayout layout_of(int T, int H, int d_v, int P) {
  WorkspaceLayout w;
  const size_t splits = (size_t)T + (size_t)P;
  w.o_acc = 0;
  w.lse_acc = round_up(w.o_acc + splits * H * d_v * sizeof(float), 256);
  w.meta = round_up(w.lse_acc + splits * H * sizeof(float), 256);
  w.num_splits = round_up(w.meta + (size_t)P * SDA_META_INTS * sizeof(int32_t), 256);
  w.total = round_up(w.num_splits + ((size_t)T + 1) * sizeof(int32_t), 256);
  w.q_rot = w.total;
  w.total_v41 = round_up(w.q_rot + (size_t)T * H * 64 * sizeof(uint16_t), 256);
  return w;
}

sda::ListDev list_dev(const sda_cache* c, const sda_list* l) {
  sda::ListDev d;
  memset(&d, 0, sizeof(d));
  d.idx = l->idx;
  d.lens = l->lens;
  d.base = (const uint8_t*)c->base;
  d.slot_scale = c->slot_scale;
  d.row_stride = l->row_stride;
  d.page_stride = c->page_stride;
  d.width = l->width;
  d.slots = (int32_t)(c->num_pages * c->page_size);
  d.page_shift = ilog2(c->page_size);
  d.format = c->format;
  d.rec = sda_record_bytes(c->format);
  d.lens_div = lens_div(l);
  return d;
}

}  // namespace

namespace sda {
hipError_t launch_decode(const DecodeParams& p, int num_parts, int heads_per_group, int d_qk, int precision,
                         hipStream_t stream) {
  const bool fp4 = p.lst[0].format == SDA_NVFP4_288 || (p.nlists > 1 && p.lst[1].format == SDA_NVFP4_288);
  // the ring kernel takes FP8_UE8M0 lists only when every list is one
  const int ue = (p.lst[0].format == SDA_FP8_UE8M0) + (p.nlists > 1 && p.lst[1].format == SDA_FP8_UE8M0);
  // MODEL1_584 lists: the ring kernel when every list is one and a workgroup takes 32 or more heads (its
  // 592-byte ring rows leave no room for two 16-head workgroups per CU), else the staged kernel
  const int m1 = (p.lst[0].format == SDA_MODEL1_584) + (p.nlists > 1 && p.lst[1].format == SDA_MODEL1_584);
  const bool staged = fp4 || (m1 > 0 && (m1 < p.nlists || heads_per_group < 32)) || (ue > 0 && ue < p.nlists);
  // 576-dim records (every list SDA_V32_656) with 64 heads per workgroup: the 32x32-product kernel
  if (d_qk == 576 && heads_per_group == 64) return launch_decode_wide(p, num_parts, precision, stream);
  // the register-staged kernel takes at most 32 heads per workgroup
  return staged ? launch_decode_staged(p, num_parts, heads_per_group > 32 ? 32 : heads_per_group, d_qk, precision,
                                       stream)
                : launch_decode_ring(p, num_parts, heads_per_group, d_qk, precision, stream);
}
}  // namespace sda

namespace {

sda::SchedParams sched_params(int T, const sda_list* list, const sda_list* extra, const sda_plan* plan, int32_t* meta,
                              int32_t* num_splits) {
  sda::SchedParams s;
  memset(&s, 0, sizeof(s));
  s.lens[0] = list->lens;
  s.lens_div[0] = lens_div(list);
  s.width[0] = list->width;
  s.nlists = 1;
  if (extra) {
    s.lens[1] = extra->lens;
    s.lens_div[1] = lens_div(extra);
    s.width[1] = extra->width;
    s.nlists = 2;
  }
  s.T = T;
  s.num_parts = plan->num_parts;
  s.F = plan->fixed_overhead;
  s.meta = meta;
  s.num_splits = num_splits;
  return s;
}

}  // namespace

namespace {

// Workspace of sda_sparse_decode_attn_noalloc: one copy per GPU, held until the process ends. Host code
// never uses this name as an address: each device's copy is reached through the address that
// hipGetSymbolAddress returns for it, with that device current.
static __device__ __align__(256) char scratch[SDA_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up on the first call on that device.
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SDA_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(SDA_ERR_HIP, "scratch symbol address missing or misaligned");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SDA_OK;
}

}  // namespace

extern "C" {

const char* sda_status_string(int status) {
  switch (status) {
    case SDA_OK: return "ok";
    case SDA_ERR_INVALID_ARG: return "invalid argument";
    case SDA_ERR_UNSUPPORTED: return "unsupported shape or format";
    case SDA_ERR_WORKSPACE: return "workspace too small";
    case SDA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sda_last_error(void) { return g_last_error; }

int sda_record_bytes(int format) {
  switch (format) {
    case SDA_FP8_SLOTSCALE: return 512;
    case SDA_FP8_528: return 528;
    case SDA_NVFP4_288: return 288;
    case SDA_V32_656: return 656;
    case SDA_FP8_UE8M0: return 528;
    case SDA_MODEL1_584: return 584;
    default: return -1;
  }
}

int sda_format_dims(int format) {
  switch (format) {
    case SDA_FP8_SLOTSCALE:
    case SDA_FP8_528:
    case SDA_NVFP4_288:
    case SDA_FP8_UE8M0:
    case SDA_MODEL1_584: return 512;
    case SDA_V32_656: return 576;
    default: return -1;
  }
}

int sda_make_plan(int T, int H, int d_qk, int width, int extra_width, int num_cus, sda_plan* plan) {
  if (!plan) return fail(SDA_ERR_INVALID_ARG, "plan is NULL");
  if (T < 1 || width < 1 || extra_width < 0) return fail(SDA_ERR_INVALID_ARG, "T and width must be >= 1");
  if (!supported_heads(H)) return fail(SDA_ERR_UNSUPPORTED, "H must be 16, 32, 64 or 128");
  if (d_qk != 512 && d_qk != 576) return fail(SDA_ERR_UNSUPPORTED, "d_qk must be 512 or 576");
  if (num_cus <= 0) num_cus = 256;
  // Heads per workgroup: 64 for 576-dim records when H allows it (eight waves, one workgroup per CU,
  // every record gathered once per 64 heads: the long top-k lists are bound by the gathers), else 32
  // when H allows it (eight waves, one workgroup per CU), else 16 (four waves; two workgroups per CU
  // for fp8 records, three for NVFP4 ones: three parts per CU). The parts fill every workgroup slot
  // once; a part's head groups land on the same XCD (shared L2) when num_parts % 8 == 0.
  const int hb = (d_qk == 576 && H >= 64) ? 64 : (H >= 32 ? 32 : 16);
  const int groups = H / hb;
  const int slots_per_cu = (hb == 16 && d_qk == 512) ? 3 : 1;
  int parts = (slots_per_cu * num_cus) / groups;
  parts = ((parts + 7) / 8) * 8;
  if (parts < 8) parts = 8;
  plan->num_parts = parts;
  plan->heads_per_group = hb;
  // per-token overhead in the cost model: 2 tiles for 32-head groups; 0 for 16-head groups, whose
  // long NVFP4 lists balance best when parts are cut by tiles alone (measured)
  plan->fixed_overhead = hb == 16 ? 0 : 2;
  plan->precision = 2;
  plan->whole_tokens = 0;
  return SDA_OK;
}

// The choice between the split plan and a whole-token plan compares the two schedules' makespans in
// 64-row tiles. One workgroup per token takes about the longest token's tiles, or the even share
// total / num_parts once tokens outnumber the split plan's parts; the split plan takes about
// (total + T x fixed overhead) / num_parts and two more launches (scheduler and combine; the V4.1 call
// keeps its epilogue, so it saves only the scheduler), each worth about a tile. The whole-token plan is
// taken while its makespan is within 1.3x the split one plus two tiles (1.0x plus one for V4.1):
// measured on MI355X, it wins where tokens are equal or a few tiles apart (the split plan also pays its
// partial writes and token switches) and loses where one long token leaves the GPU idle.
int sda_choose_plan(int T, int H, int d_qk, int format, const int32_t* lens, int width, int extra_format,
                    const int32_t* extra_lens, int extra_width, int queries_per_len, int v41, int num_cus,
                    sda_plan* plan) {
  if (!plan) return fail(SDA_ERR_INVALID_ARG, "plan is NULL");
  if (queries_per_len < 0) return fail(SDA_ERR_INVALID_ARG, "queries_per_len must be >= 0");
  if (sda_record_bytes(format) < 0 || sda_format_dims(format) != d_qk)
    return fail(SDA_ERR_UNSUPPORTED, "main list format unknown or not of d_qk dims");
  const bool has_extra = extra_width > 0;
  if (has_extra && (sda_record_bytes(extra_format) < 0 || sda_format_dims(extra_format) != d_qk))
    return fail(SDA_ERR_UNSUPPORTED, "extra list format unknown or not of d_qk dims");
  if (!has_extra && extra_lens) return fail(SDA_ERR_INVALID_ARG, "extra_lens without an extra list");
  int rc = sda_make_plan(T, H, d_qk, width, has_extra ? extra_width : 0, num_cus, plan);
  if (rc) return rc;
  if (num_cus <= 0) num_cus = 256;
  const int div = queries_per_len > 1 ? queries_per_len : 1;
  int64_t total = 0, longest = 0;
  for (int t = 0; t < T; ++t) {
    const int n0 = sda::clamp_len(lens, div, width, t);
    const int n1 = has_extra ? sda::clamp_len(extra_lens, div, extra_width, t) : 0;
    const int64_t nt = sda::token_tiles(n0, n1);
    total += nt;
    if (nt > longest) longest = nt;
  }
  const int64_t share = (total + plan->num_parts - 1) / plan->num_parts;
  const double whole = (double)(longest > share ? longest : share);
  const double split = (double)(total + (int64_t)T * plan->fixed_overhead) / plan->num_parts;
  const double ratio = v41 ? 1.0 : 1.3, slack = v41 ? 1.0 : 2.0;
  if (!(whole <= ratio * split + slack)) return SDA_OK;
  plan->whole_tokens = 1;
  // 16 heads per workgroup where the call runs the fp8 ring kernel on 512-dim records (no NVFP4 or MODEL1
  // list; FP8_UE8M0 lists only with one another) and T x H/16 workgroups fit one round of two per CU: the
  // four-wave workgroups overlap one another's gathers (measured 1.6-3.7 % faster steps than 32-head
  // workgroups). MODEL1 lists run the ring kernel only with 32 or more heads per workgroup.
  const int fm[2] = {format, has_extra ? extra_format : -1};
  const int nf = has_extra ? 2 : 1;
  int ue = 0;
  bool ring = true;
  for (int i = 0; i < nf; ++i) {
    ue += fm[i] == SDA_FP8_UE8M0;
    if (fm[i] == SDA_NVFP4_288 || fm[i] == SDA_MODEL1_584) ring = false;
  }
  if (ue != 0 && ue != nf) ring = false;
  if (d_qk == 512 && ring && plan->heads_per_group == 32 && (int64_t)T * (H / 16) <= 2 * (int64_t)num_cus)
    plan->heads_per_group = 16;
  return SDA_OK;
}

size_t sda_workspace_bytes(int T, int H, int d_v, const sda_plan* plan) {
  if (!plan || T < 1 || H < 1 || d_v < 1 || plan->num_parts < 1) return 0;
  return layout_of(T, H, d_v, plan->num_parts).total;
}

int sda_get_sched_meta(int T, const sda_list* list, const sda_list* extra, const sda_plan* plan, int32_t* meta,
                       int32_t* num_splits, void* stream) {
  if (T < 1) return fail(SDA_ERR_INVALID_ARG, "T must be >= 1");
  int rc = check_list(list, "main");
  if (rc) return rc;
  if (extra && (rc = check_list(extra, "extra"))) return rc;
  if (!plan || plan->num_parts < 1 || plan->fixed_overhead < 0) return fail(SDA_ERR_INVALID_ARG, "bad plan");
  if (plan->whole_tokens) return fail(SDA_ERR_INVALID_ARG, "a whole-token plan has no schedule");
  if (!meta || !num_splits) return fail(SDA_ERR_INVALID_ARG, "meta and num_splits are required");
  if ((rc = check_cost_range(T, list->width, extra ? extra->width : 0, plan))) return rc;
  hipError_t e = sda::launch_sched(sched_params(T, list, extra, plan, meta, num_splits), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sched kernel launch");
  return SDA_OK;
}

int sda_get_sched_meta_host(int T, int queries_per_len, const int32_t* lens, int width, const int32_t* extra_lens,
                            int extra_width, const sda_plan* plan, int32_t* meta, int32_t* num_splits) {
  if (T < 1 || width < 1 || extra_width < 0) return fail(SDA_ERR_INVALID_ARG, "T and width must be >= 1");
  if (queries_per_len < 0) return fail(SDA_ERR_INVALID_ARG, "queries_per_len must be >= 0");
  const int div = queries_per_len > 1 ? queries_per_len : 1;
  if (!plan || plan->num_parts < 1 || plan->fixed_overhead < 0) return fail(SDA_ERR_INVALID_ARG, "bad plan");
  if (plan->whole_tokens) return fail(SDA_ERR_INVALID_ARG, "a whole-token plan has no schedule");
  if (!meta || !num_splits) return fail(SDA_ERR_INVALID_ARG, "meta and num_splits are required");
  if (int rc = check_cost_range(T, width, extra_width, plan)) return rc;
  const int P = plan->num_parts, F = plan->fixed_overhead;
  int64_t total = 0;
  for (int t = 0; t < T; ++t) {
    const int n0 = sda::clamp_len(lens, div, width, t);
    const int n1 = extra_width > 0 ? sda::clamp_len(extra_lens, div, extra_width, t) : 0;
    total += sda::token_tiles(n0, n1) + F;
  }
  const int64_t Q = sda::part_quantum(total, P);
  int64_t cum = 0;
  int32_t splits = 0;
  for (int t = 0; t < T; ++t) {
    const int n0 = sda::clamp_len(lens, div, width, t);
    const int n1 = extra_width > 0 ? sda::clamp_len(extra_lens, div, extra_width, t) : 0;
    const int nt = sda::token_tiles(n0, n1);
    const int64_t pos0 = cum + F;
    const int64_t p0 = pos0 / Q, p1 = (pos0 + nt - 1) / Q;
    num_splits[t] = splits;
    splits += (int32_t)(p1 - p0 + 1);
    const int64_t prev_last = (cum == 0) ? -1 : (cum - 1) / Q;
    for (int64_t pp = prev_last + 1; pp <= p1; ++pp) {
      const int64_t bi = pp * Q - pos0 > 0 ? pp * Q - pos0 : 0;
      int32_t* m = meta + pp * SDA_META_INTS;
      m[0] = t;
      m[1] = (int32_t)bi;
      m[4] = pp >= p0 ? (int32_t)(pp - p0) : 0;
      m[5] = n0;
      m[6] = n1;
      m[7] = num_splits[t];
      if (pp > 0) {
        meta[(pp - 1) * SDA_META_INTS + 2] = t;
        meta[(pp - 1) * SDA_META_INTS + 3] = (int32_t)bi;
      }
    }
    cum += nt + F;
  }
  num_splits[T] = splits;
  const int64_t last = (total - 1) / Q;
  for (int64_t pp = last + 1; pp < P; ++pp) {
    int32_t* m = meta + pp * SDA_META_INTS;
    m[0] = T; m[1] = 0; m[2] = T; m[3] = 0; m[4] = 0; m[5] = 0; m[6] = 0; m[7] = 0;
  }
  meta[last * SDA_META_INTS + 2] = T;
  meta[last * SDA_META_INTS + 3] = 0;
  return SDA_OK;
}

namespace {

// Checks shared by sda_sparse_decode_attn and sda_decode_splits.
int check_decode_args(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
                      const sda_cache* cache, const sda_list* list, const sda_cache* extra_cache,
                      const sda_list* extra_list, const sda_plan* plan, const int32_t* meta, const int32_t* num_splits,
                      void* workspace, size_t workspace_bytes, void* out, int64_t out_stride_t, int64_t out_stride_h,
                      float* lse, int64_t lse_stride_t, bool no_out = false, bool v41 = false,
                      bool noalloc = false) {
  // no_out: no bf16 output and an optional lse (V4.1 calls, whose fp8 output is checked by the caller, and
  // decode-only calls that leave every token as a partial)
  if (!q) return fail(SDA_ERR_INVALID_ARG, "q is required");
  if (!no_out && (!out || !lse)) return fail(SDA_ERR_INVALID_ARG, "q, out and lse are required");
  if (T < 1) return fail(SDA_ERR_INVALID_ARG, "T must be >= 1");
  if (!supported_heads(H)) return fail(SDA_ERR_UNSUPPORTED, "H must be 16, 32, 64 or 128");
  if (!((d_qk == 512 || d_qk == 576) && d_v == 512))
    return fail(SDA_ERR_UNSUPPORTED, "(d_qk, d_v) must be (512, 512) or (576, 512)");
  if (!aligned(q, 16) || q_stride_h % 8 || q_stride_t % 8 || q_stride_h < d_qk || q_stride_t < 0)
    return fail(SDA_ERR_INVALID_ARG, "q must be 16-byte aligned with strides that are multiples of 8 elements");
  if (!no_out && (!aligned(out, 16) || out_stride_h % 8 || out_stride_t % 8 || out_stride_h < d_v || out_stride_t < 0))
    return fail(SDA_ERR_INVALID_ARG, "out must be 16-byte aligned with strides that are multiples of 8 elements");
  if (lse && lse_stride_t < H) return fail(SDA_ERR_INVALID_ARG, "lse_stride_t must be >= H");
  int rc;
  if ((rc = check_cache(cache, d_qk, "main"))) return rc;
  if ((rc = check_list(list, "main"))) return rc;
  if ((extra_cache == nullptr) != (extra_list == nullptr))
    return fail(SDA_ERR_INVALID_ARG, "extra_cache and extra_list must be given together");
  if (extra_cache) {
    if ((rc = check_cache(extra_cache, d_qk, "extra"))) return rc;
    if ((rc = check_list(extra_list, "extra"))) return rc;
  }
  if ((rc = check_plan(plan, H))) return rc;
  if (!plan->whole_tokens &&
      (rc = check_cost_range(T, list->width, extra_list ? extra_list->width : 0, plan)))
    return rc;
  if ((meta == nullptr) != (num_splits == nullptr))
    return fail(SDA_ERR_INVALID_ARG, "meta and num_splits must be given together");
  if (plan->whole_tokens && meta)
    return fail(SDA_ERR_INVALID_ARG, "a whole-token plan reads no meta or num_splits: pass NULL for both");
  const WorkspaceLayout wl = layout_of(T, H, d_v, plan->num_parts);
  if (!workspace || !aligned(workspace, 256)) return fail(SDA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  // noalloc: the static scratch, checked against what the call touches (nothing for a whole-token plan)
  const size_t need = noalloc ? (plan->whole_tokens ? 0 : wl.total) : (v41 ? wl.total_v41 : wl.total);
  if (noalloc && workspace_bytes < need)
    return fail(SDA_ERR_WORKSPACE, "the plan's workspace exceeds SDA_SCRATCH_BYTES");
  if (workspace_bytes < need)
    return fail(SDA_ERR_WORKSPACE, v41 ? "workspace smaller than sda_workspace_bytes_v41()"
                                       : "workspace smaller than sda_workspace_bytes()");
  return SDA_OK;
}

int check_v41(const sda_v41* v, int T, int H) {
  if (!v) return fail(SDA_ERR_INVALID_ARG, "v41 descriptor is NULL");
  if (!v->positions || !v->cos_sin || !v->out_fp8 || !v->out_scale)
    return fail(SDA_ERR_INVALID_ARG, "v41: positions, cos_sin, out_fp8 and out_scale are required");
  if (!aligned(v->positions, 8) || !aligned(v->cos_sin, 16) || v->cs_stride < 64 || v->cs_stride % 4 ||
      v->num_positions < 0)
    return fail(SDA_ERR_INVALID_ARG, "v41: cos_sin must be 16-byte aligned with a stride >= 64 and a multiple of 4");
  if (!aligned(v->out_fp8, 16) || v->of_stride_h < 512 || v->of_stride_h % 16 || v->of_stride_t < 0 ||
      v->of_stride_t % 16)
    return fail(SDA_ERR_INVALID_ARG, "v41: out_fp8 must be 16-byte aligned with strides in 16s, of_stride_h >= 512");
  if (v->os_stride_h < 16 || v->os_stride_t < 0)
    return fail(SDA_ERR_INVALID_ARG, "v41: os_stride_h must be >= 16");
  (void)T;
  (void)H;
  return SDA_OK;
}

// Workgroups along the grid's first dimension: the scheduler's parts, or one per token (whole-token plans).
int grid_parts(const sda_plan* plan, int T) { return plan->whole_tokens ? T : plan->num_parts; }

sda::DecodeParams decode_params(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H,
                                const sda_cache* cache, const sda_list* list, const sda_cache* extra_cache,
                                const sda_list* extra_list, const float* attn_sink, float scale, const int32_t* meta,
                                const int32_t* num_splits, char* ws, const WorkspaceLayout& wl, void* out,
                                int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t) {
  sda::DecodeParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const uint16_t*)q;
  p.q_st = q_stride_t;
  p.q_sh = q_stride_h;
  p.out = (uint16_t*)out;
  p.o_st = out_stride_t;
  p.o_sh = out_stride_h;
  p.lse = lse;
  p.l_st = lse_stride_t;
  p.sink = attn_sink;
  p.meta = meta;
  p.num_splits = num_splits;
  p.o_acc = (float*)(ws + wl.o_acc);
  p.lse_acc = (float*)(ws + wl.lse_acc);
  p.lst[0] = list_dev(cache, list);
  p.nlists = 1;
  if (extra_cache) {
    p.lst[1] = list_dev(extra_cache, extra_list);
    p.nlists = 2;
  }
  p.T = T;
  p.H = H;
  p.scale_log2 = scale * 1.4426950408889634f;
  return p;
}

sda::CombineParams combine_params(int T, int H, const float* o_acc, const float* lse_acc, const int32_t* num_splits,
                                  const float* attn_sink, void* out, int64_t out_stride_t, int64_t out_stride_h,
                                  float* lse, int64_t lse_stride_t) {
  sda::CombineParams c;
  memset(&c, 0, sizeof(c));
  c.o_acc = o_acc;
  c.lse_acc = lse_acc;
  c.num_splits = num_splits;
  c.sink = attn_sink;
  c.out = (uint16_t*)out;
  c.o_st = out_stride_t;
  c.o_sh = out_stride_h;
  c.lse = lse;
  c.l_st = lse_stride_t;
  c.T = T;
  c.H = H;
  return c;
}

}  // namespace

size_t sda_workspace_lse_offset(int T, int H, int d_v, const sda_plan* plan) {
  if (!plan || T < 1 || H < 1 || d_v < 1 || plan->num_parts < 1) return 0;
  return layout_of(T, H, d_v, plan->num_parts).lse_acc;
}

int sda_decode_splits(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
                      const sda_cache* cache, const sda_list* list, const sda_cache* extra_cache,
                      const sda_list* extra_list, const float* attn_sink, float scale, const sda_plan* plan,
                      const int32_t* meta, const int32_t* num_splits, void* workspace, size_t workspace_bytes,
                      void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                      void* stream) {
  // out NULL: every token leaves as a partial in the workspace (lse is then not used)
  const bool no_out = out == nullptr;
  int rc = check_decode_args(q, q_stride_t, q_stride_h, T, H, d_qk, d_v, cache, list, extra_cache, extra_list, plan,
                             meta, num_splits, workspace, workspace_bytes, out, out_stride_t, out_stride_h, lse,
                             lse_stride_t, no_out);
  if (rc) return rc;
  if (!meta && !plan->whole_tokens) return fail(SDA_ERR_INVALID_ARG, "sda_decode_splits needs meta and num_splits");
  const WorkspaceLayout wl = layout_of(T, H, d_v, plan->num_parts);
  sda::DecodeParams p = decode_params(q, q_stride_t, q_stride_h, T, H, cache, list, extra_cache, extra_list,
                                      attn_sink, scale, meta, num_splits, (char*)workspace, wl, out, out_stride_t,
                                      out_stride_h, no_out ? nullptr : lse, lse_stride_t);
  p.all_partial = no_out ? 1 : 0;
  hipError_t e = sda::launch_decode(p, grid_parts(plan, T), plan->heads_per_group, d_qk, plan->precision,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  return SDA_OK;
}

}  // extern "C"

namespace {

// The whole op; noalloc: the workspace is the static scratch (checked against what the plan touches).
int decode_attn_impl(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
                     const sda_cache* cache, const sda_list* list, const sda_cache* extra_cache,
                     const sda_list* extra_list, const float* attn_sink, float scale, const sda_plan* plan,
                     const int32_t* meta, const int32_t* num_splits, void* workspace, size_t workspace_bytes,
                     void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                     void* stream, bool noalloc) {
  int rc = check_decode_args(q, q_stride_t, q_stride_h, T, H, d_qk, d_v, cache, list, extra_cache, extra_list, plan,
                             meta, num_splits, workspace, workspace_bytes, out, out_stride_t, out_stride_h, lse,
                             lse_stride_t, false, false, noalloc);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const WorkspaceLayout wl = layout_of(T, H, d_v, plan->num_parts);
  if (!meta && !plan->whole_tokens) {
    int32_t* m = (int32_t*)(ws + wl.meta);
    int32_t* ns = (int32_t*)(ws + wl.num_splits);
    hipError_t e = sda::launch_sched(sched_params(T, list, extra_list, plan, m, ns), st);
    if (e != hipSuccess) return hip_fail(e, "sched kernel launch");
    meta = m;
    num_splits = ns;
  }
  const sda::DecodeParams p = decode_params(q, q_stride_t, q_stride_h, T, H, cache, list, extra_cache, extra_list,
                                            attn_sink, scale, meta, num_splits, ws, wl, out, out_stride_t,
                                            out_stride_h, lse, lse_stride_t);
  hipError_t e = sda::launch_decode(p, grid_parts(plan, T), plan->heads_per_group, d_qk, plan->precision, st);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  if (plan->whole_tokens) return SDA_OK;  // every token was written whole by the decode kernel
  e = sda::launch_combine(combine_params(T, H, p.o_acc, p.lse_acc, num_splits, attn_sink, out, out_stride_t,
                                         out_stride_h, lse, lse_stride_t),
                          st);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return SDA_OK;
}

}  // namespace

extern "C" {

int sda_sparse_decode_attn(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
                           const sda_cache* cache, const sda_list* list, const sda_cache* extra_cache,
                           const sda_list* extra_list, const float* attn_sink, float scale, const sda_plan* plan,
                           const int32_t* meta, const int32_t* num_splits, void* workspace, size_t workspace_bytes,
                           void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                           void* stream) {
  return decode_attn_impl(q, q_stride_t, q_stride_h, T, H, d_qk, d_v, cache, list, extra_cache, extra_list, attn_sink,
                          scale, plan, meta, num_splits, workspace, workspace_bytes, out, out_stride_t, out_stride_h,
                          lse, lse_stride_t, stream, false);
}

size_t sda_noalloc_workspace_bytes(int T, int H, int d_v, const sda_plan* plan) {
  if (!plan || T < 1 || H < 1 || d_v < 1 || plan->num_parts < 1) return 0;
  // a whole-token plain call writes every token whole: no partials, no schedule
  return plan->whole_tokens ? 0 : layout_of(T, H, d_v, plan->num_parts).total;
}

int sda_sparse_decode_attn_noalloc(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk,
                                   int d_v, const sda_cache* cache, const sda_list* list,
                                   const sda_cache* extra_cache, const sda_list* extra_list, const float* attn_sink,
                                   float scale, const sda_plan* plan, const int32_t* meta, const int32_t* num_splits,
                                   void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse,
                                   int64_t lse_stride_t, void* stream) {
  if (!plan) return fail(SDA_ERR_INVALID_ARG, "plan is NULL");
  if (T < 1 || H < 1 || d_v < 1 || plan->num_parts < 1) return fail(SDA_ERR_INVALID_ARG, "T, H, d_v and num_parts must be >= 1");
  const size_t need = sda_noalloc_workspace_bytes(T, H, d_v, plan);
  if (need > (size_t)SDA_SCRATCH_BYTES)
    return fail(SDA_ERR_WORKSPACE, "the plan's workspace exceeds SDA_SCRATCH_BYTES (use a whole-token plan, fewer "
                                   "parts or tokens, or sda_sparse_decode_attn with a caller workspace)");
  void* ws = nullptr;
  int rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  return decode_attn_impl(q, q_stride_t, q_stride_h, T, H, d_qk, d_v, cache, list, extra_cache, extra_list, attn_sink,
                          scale, plan, meta, num_splits, ws, (size_t)SDA_SCRATCH_BYTES, out, out_stride_t,
                          out_stride_h, lse, lse_stride_t, stream, true);
}

int sda_combine_splits(int T, int H, int d_v, const float* o_accum, const float* lse_accum, const int32_t* num_splits,
                       const float* attn_sink, void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse,
                       int64_t lse_stride_t, void* stream) {
  if (T < 1) return fail(SDA_ERR_INVALID_ARG, "T must be >= 1");
  // the combine kernel computes 16 heads per workgroup (one wave each) and stores 8 bf16 per lane
  if (!supported_heads(H)) return fail(SDA_ERR_UNSUPPORTED, "H must be 16, 32, 64 or 128");
  if (d_v != 512) return fail(SDA_ERR_UNSUPPORTED, "d_v must be 512");
  if (!o_accum || !lse_accum || !num_splits || !out || !lse) return fail(SDA_ERR_INVALID_ARG, "NULL buffer");
  if (!aligned(o_accum, 16) || !aligned(out, 16) || out_stride_h % 8 || out_stride_t % 8 || out_stride_h < d_v ||
      out_stride_t < 0)
    return fail(SDA_ERR_INVALID_ARG,
                "o_accum and out must be 16-byte aligned, out strides multiples of 8 elements");
  if (lse_stride_t < H) return fail(SDA_ERR_INVALID_ARG, "lse_stride_t must be >= H");
  const sda::CombineParams c = combine_params(T, H, o_accum, lse_accum, num_splits, attn_sink, out, out_stride_t,
                                             out_stride_h, lse, lse_stride_t);
  hipError_t e = sda::launch_combine(c, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return SDA_OK;
}


size_t sda_workspace_bytes_v41(int T, int H, const sda_plan* plan) {
  if (!plan || T < 1 || H < 1 || plan->num_parts < 1) return 0;
  return layout_of(T, H, 512, plan->num_parts).total_v41;
}

int sda_sparse_decode_attn_v41(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H,
                               const sda_cache* cache, const sda_list* list, const sda_cache* extra_cache,
                               const sda_list* extra_list, const float* attn_sink, float scale, const sda_plan* plan,
                               const int32_t* meta, const int32_t* num_splits, void* workspace,
                               size_t workspace_bytes, const sda_v41* v41, float* lse, int64_t lse_stride_t,
                               void* stream) {
  int rc = check_decode_args(q, q_stride_t, q_stride_h, T, H, 512, 512, cache, list, extra_cache, extra_list, plan,
                             meta, num_splits, workspace, workspace_bytes, nullptr, 0, 0, lse, lse_stride_t, true, true);
  if (rc) return rc;
  if ((rc = check_v41(v41, T, H))) return rc;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const WorkspaceLayout wl = layout_of(T, H, 512, plan->num_parts);
  if (!meta && !plan->whole_tokens) {
    int32_t* m = (int32_t*)(ws + wl.meta);
    int32_t* ns = (int32_t*)(ws + wl.num_splits);
    hipError_t e = sda::launch_sched(sched_params(T, list, extra_list, plan, m, ns), st);
    if (e != hipSuccess) return hip_fail(e, "sched kernel launch");
    meta = m;
    num_splits = ns;
  }
  // prologue: q with its RoPE dims rotated, into the workspace
  sda::RopeParams rp;
  memset(&rp, 0, sizeof(rp));
  rp.q = (const uint16_t*)q;
  rp.q_st = q_stride_t;
  rp.q_sh = q_stride_h;
  rp.q_out = (uint16_t*)(ws + wl.q_rot);
  rp.positions = v41->positions;
  rp.cos_sin = v41->cos_sin;
  rp.cs_stride = v41->cs_stride;
  rp.num_positions = v41->num_positions;
  rp.T = T;
  rp.H = H;
  hipError_t e = sda::launch_rope_q(rp, st);
  if (e != hipSuccess) return hip_fail(e, "rope kernel launch");
  // decode on q with its rotated dims from the workspace, every token leaving as an fp32 partial
  sda::DecodeParams p = decode_params(q, q_stride_t, q_stride_h, T, H, cache, list, extra_cache, extra_list,
                                      attn_sink, scale, meta, num_splits, ws, wl, nullptr, 0, 0, nullptr, 0);
  p.q_rope = rp.q_out;
  p.all_partial = 1;
  e = sda::launch_decode(p, grid_parts(plan, T), plan->heads_per_group, 512, plan->precision, st);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  // combine every token: merge, inverse RoPE, MXFP8
  sda::CombineParams c = combine_params(T, H, p.o_acc, p.lse_acc, num_splits, attn_sink, nullptr, 0, 0, lse,
                                        lse_stride_t);
  c.positions = v41->positions;
  c.cos_sin = v41->cos_sin;
  c.cs_stride = v41->cs_stride;
  c.num_positions = v41->num_positions;
  c.o8 = v41->out_fp8;
  c.o8_st = v41->of_stride_t;
  c.o8_sh = v41->of_stride_h;
  c.osc = v41->out_scale;
  c.osc_st = v41->os_stride_t;
  c.osc_sh = v41->os_stride_h;
  e = sda::launch_combine(c, st);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return SDA_OK;
}

}  // extern "C"
