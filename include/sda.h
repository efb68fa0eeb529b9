/* sda.h -- C ABI of the MI355X (gfx950) decode-attention library for paged,
 * quantized, shared-KV caches ("sparse decode attention").
 *
 * One decode step: for every decode token t and query head h, gather latent
 * KV rows by slot id from a paged cache, dequantize them, use each row as both
 * key (all d_qk dims) and value (its first d_v = 512 dims), run a softmax with
 * an optional per-head attention-sink logit, and write a bf16 output plus the
 * fp32 log-sum-exp. The rows of a token come from a main slot list (a sliding
 * window or a top-k list) followed by an optional "extra" list (compressed
 * cache). Work is split across the GPU by a scheduler and merged by LSE.
 *
 * Sources of each operation (page titles as they appear online):
 *  - interface, feature set and checks: FlashMLA csrc/api/sparse_decode.h,
 *    sparse_attn_decode_interface (argument list, validation, outputs) and the
 *    DecodeImplMeta / get_meta scheduler parameters;
 *  - gather, validity and page addressing: vLLM swapab_decode_attn,
 *    stage_inputs and the __call__ contract;
 *  - sink and LSE merge: vLLM swapab_decode_attn device kernel, step 9;
 *    dsv4 production.py, _run_fmha_segmented (segment merge);
 *  - per-slot fp8 dequant: native_swa_decode.py, native_swa_decode_attention.
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless marked (host). The caller allocates and
 *    owns every buffer; the library allocates nothing and keeps no pointer after
 *    a call returns. Device buffers must stay valid until `stream` has run the
 *    work.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on it; none synchronizes the device.
 *  - Return value: 0 (SDA_OK) or a negative sda_status. Problems detectable on
 *    the host return an error and enqueue nothing. Data held in device memory is
 *    never an error: slot ids < 0 or >= the cache's slot count, and list
 *    positions at or past a token's length, are masked; lengths are clamped to
 *    [0, width].
 *  - No entry point aborts the process or throws.
 */
#ifndef SDA_H
#define SDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum sda_status {
  SDA_OK = 0,
  SDA_ERR_INVALID_ARG = -1,  /* NULL pointer, bad size, misaligned buffer, inconsistent lists      */
  SDA_ERR_UNSUPPORTED = -2,  /* head count, head dims or format combination not supported          */
  SDA_ERR_WORKSPACE = -3,    /* workspace too small for the plan                                  */
  SDA_ERR_HIP = -4           /* a HIP launch failed; sda_last_error() has the runtime's message    */
};

/* Cache record formats (bytes of one slot).
 * SDA_FP8_SLOTSCALE  512 B: 512 e4m3fn codes; the scale is slot_scale[slot_id] (fp32), multiplied
 *                    into the row (native_swa_decode.py: batched gather + dequant pre-step).
 * SDA_FP8_528        528 B: 512 e4m3fn codes, then 4 little-endian fp32 scales, scale g covering
 *                    dims [128g, 128g+128).
 * SDA_NVFP4_288      288 B: 256 bytes of packed e2m1 (the low nibble of byte i is dim 2i, the high
 *                    nibble dim 2i+1), then 32 e4m3fn block scales, scale b covering dims
 *                    [16b, 16b+16) (vLLM swapab_decode_attn, stage_inputs, NVFP4 branch).
 * SDA_V32_656        656 B: as SDA_FP8_528 for dims 0..511, then 64 little-endian bf16 values for
 *                    dims 512..575 (FlashMLA sparse_decode.h: V3.2 bytes_per_token); d_qk = 576.
 * SDA_FP8_UE8M0      528 B: 512 e4m3fn codes, then 16 ue8m0 scale bytes, byte g the power of two
 *                    2^(g - 127) covering dims [32g, 32g+32) (vLLM swapab_decode_attn, stage_inputs,
 *                    fp8 branch); byte 255 (NaN in the MX encoding) gives NaN rows.
 * SDA_MODEL1_584     584 B, d_qk = d_v = 512: 448 e4m3fn codes (dims 0..447), 64 little-endian bf16
 *                    values (dims 448..511), 7 ue8m0 scale bytes (byte g covering dims [64g, 64g+64)),
 *                    one unused byte (FlashMLA sparse_decode.h: MODEL1 bytes_per_token; the page gives
 *                    the parts and their sum, and they are laid out in the order of that sum). The
 *                    value rows are the whole 512 dims, the bf16 ones included. Records start 8-byte
 *                    aligned.
 * A decoded value is code * scale (exact in bf16 for every format; for the ue8m0 formats while it
 * stays within the bf16 range). */
enum sda_format { SDA_FP8_SLOTSCALE = 0, SDA_FP8_528 = 1, SDA_NVFP4_288 = 2, SDA_V32_656 = 3, SDA_FP8_UE8M0 = 4,
                  SDA_MODEL1_584 = 5 };

/* A paged cache. Slot id s lives in page s / page_size at offset s % page_size; its record starts
 * at base + (s / page_size) * page_stride + (s % page_size) * record_bytes. Pages may be further
 * apart than page_size * record_bytes (vLLM swapab_decode_attn, __call__ contract).
 * Requirements: base 16-byte aligned, page_size a power of two, page_stride a multiple of 16 and
 * >= page_size * record_bytes, num_pages * page_size < 2^31. slot_scale: [num_pages * page_size]
 * fp32, only for SDA_FP8_SLOTSCALE (must be NULL otherwise). */
typedef struct sda_cache {
  const void* base;
  int64_t num_pages;
  int32_t page_size;
  int32_t format;
  int64_t page_stride;
  const float* slot_scale;
} sda_cache;

/* A per-token slot list: idx[t * row_stride + j] for j < width is the slot id at list position j of
 * token t (-1 = none); lens[t / queries_per_len] (or width when lens is NULL) is the number of leading
 * positions that take part. row_stride >= width; metadata buffers may hold more rows than tokens.
 * queries_per_len: consecutive tokens that share one length entry -- the s_q queries of a request
 * when q is [b][s_q][H][d] and the lengths are per request [b] (FlashMLA sparse_decode.h,
 * sparse_attn_decode_interface: topk_length [b] with indices [b][s_q][topk]); 0 or 1: one entry per
 * token. Negative values are an error. */
typedef struct sda_list {
  const int32_t* idx;
  int64_t row_stride;
  int32_t width;
  int32_t queries_per_len;
  const int32_t* lens;
} sda_list;

/* How one decode call is cut across the GPU. Filled by sda_make_plan (host only, no device access);
 * callers may adjust num_parts (>= 1) and heads_per_group (16, 32 or 64, dividing H; calls with an
 * NVFP4 list use at most 32) for tuning -- results do not depend on either beyond fp32 summation order.
 *  num_parts        scheduler parts: rows of the meta array (FlashMLA DecodeImplMeta.num_sm_parts)
 *  heads_per_group  query heads one workgroup computes; the grid is num_parts x H/heads_per_group
 *  fixed_overhead   scheduler cost of starting a token inside a part, in 64-row tiles
 *                   (DecodeImplMeta.fixed_overhead_num_blocks)
 *  precision        number of bf16 terms the softmax weights P are split into for the bf16 P.V
 *                   product: 1 = P rounded once to bf16 (fastest; ~2^-9 relative error per weight,
 *                   which can move bf16 outputs of magnitude >= 2 by one ulp, 2^-6, more often than
 *                   the 1e-2 output tolerance allows), 2 = hi + lo terms (the default; ~2^-17), 3 =
 *                   three terms whose sum is P exactly (fp32-accurate). Terms multiply the P.V
 *                   matrix-core work.
 *  whole_tokens     0 (what sda_make_plan sets): the scheduler cuts the (token, tile) sequence into
 *                   num_parts parts of equal cost, splitting tokens across parts, and a combine merges
 *                   the splits. 1: one workgroup per (token, head group) computes the token whole, in
 *                   a grid of T x H/heads_per_group; no scheduler runs, no meta or num_splits array is
 *                   read or written (callers pass NULL for both), no token is split and the plain call
 *                   runs no combine (the V4.1 call still runs its epilogue). num_parts and
 *                   fixed_overhead then only size the workspace. Results are the same either way; the
 *                   whole-token plan saves two kernel launches per call and balances the GPU when every
 *                   token has the same number of 64-row tiles (a full sliding window, a fixed top-k) and
 *                   T x H/heads_per_group fills the GPU; with uneven tokens a part may wait for the
 *                   longest. */
typedef struct sda_plan {
  int32_t num_parts;
  int32_t heads_per_group;
  int32_t fixed_overhead;
  int32_t precision;
  int32_t whole_tokens;
} sda_plan;

/* Size of one scheduler meta record, in int32 (meta is [num_parts][SDA_META_INTS]). */
#define SDA_META_INTS 8

/* Host only. Choose a plan for T tokens, H heads (16, 32, 64 or 128), d_qk (512 or 576), main list
 * width and extra list width (0 when absent), on a GPU with num_cus compute units (256 on MI355X;
 * <= 0 selects 256). Returns SDA_OK or an error for unsupported shapes. */
int sda_make_plan(int T, int H, int d_qk, int width, int extra_width, int num_cus, sda_plan* plan /*host*/);

/* Host only. The plan for a call whose token lengths the caller holds on the host (a serving engine
 * keeps them there): sda_make_plan's split plan, or a whole-token plan where the two schedules'
 * makespans, counted in 64-row tiles from these lengths, say it is faster (the FlashMLA
 * sparse_decode.h page's get_meta / DecodeImplMeta: the library picks the scheduler parameters).
 *  format, extra_format   record format of each list (extra_format ignored when extra_width is 0)
 *  lens, extra_lens       host int32 lengths, one per queries_per_len tokens as in sda_list, or NULL =
 *                         the width; extra_lens must be NULL when extra_width is 0
 *  v41                    nonzero for sda_sparse_decode_attn_v41, whose epilogue runs either way
 * The whole-token plan is taken while its makespan (the longest token, or the even share of the tiles
 * over num_parts when tokens outnumber parts) is within 1.3x the split plan's (tiles plus
 * fixed_overhead per token, over num_parts) plus two tiles for the two launches it saves (1.0x plus one
 * for V4.1); it then takes 16 heads per workgroup instead of 32 on calls whose lists are all 512-dim fp8
 * records of the fp32-scale or ue8m0 kinds when T x H/16 workgroups fit two per compute unit. Results
 * do not depend on the choice beyond fp32 summation order. Errors as sda_make_plan, plus unknown
 * formats or formats whose dims differ from d_qk. */
int sda_choose_plan(int T, int H, int d_qk, int format, const int32_t* lens /*host, nullable*/, int width,
                    int extra_format, const int32_t* extra_lens /*host, nullable*/, int extra_width,
                    int queries_per_len, int v41, int num_cus, sda_plan* plan /*host*/);

/* Host only. Bytes of workspace sda_sparse_decode_attn needs for this plan: the fp32 split partials
 * o_accum [T + num_parts][H][d_v] and lse_accum [T + num_parts][H] (FlashMLA sparse_decode.h:
 * total_num_splits = b + num_sm_parts), plus room for the meta arrays when the caller passes none. */
size_t sda_workspace_bytes(int T, int H, int d_v, const sda_plan* plan /*host*/);

/* Scheduler (FlashMLA sparse_decode.h: get_decoding_sched_meta, run when no metadata is passed in).
 * Reads the token lengths on the device, gives every token max(1, ceil(n_main/64) + ceil(n_extra/64))
 * tiles of 64 list positions plus plan->fixed_overhead, and cuts the concatenated (token, tile)
 * sequence into plan->num_parts contiguous parts of near-equal cost.
 * Writes meta [num_parts][SDA_META_INTS] int32:
 *   {begin_token, begin_tile, end_token, end_tile, begin_split, n_main, n_extra, first_split}
 * (a part covers the tiles from (begin_token, begin_tile) up to, not including, (end_token,
 * end_tile); begin_split is the index of this part among the parts that touch begin_token; n_main
 * and n_extra are begin_token's list lengths clamped to [0, width] and first_split is
 * num_splits[begin_token]; parts with no tiles hold {T, 0, T, 0, 0, 0, 0, 0}) and
 * num_splits [T+1] int32, the exclusive prefix sum of the number of parts that touch each token.
 * The result depends only on the lengths, so one call can serve every layer of a decode step.
 * extra may be NULL. A whole-token plan has no schedule: SDA_ERR_INVALID_ARG. Tile positions are
 * counted in 32-bit integers: T x (ceil(width/64) + ceil(extra_width/64) + 1 + fixed_overhead) at or
 * above 2^31 gives SDA_ERR_UNSUPPORTED. */
int sda_get_sched_meta(int T, const sda_list* list /*host*/, const sda_list* extra /*host, nullable*/,
                       const sda_plan* plan /*host*/, int32_t* meta, int32_t* num_splits, void* stream);

/* Host only. The same schedule as sda_get_sched_meta, computed on the calling thread from host
 * copies of the lengths (lens / extra_lens: one int32 per queries_per_len tokens, as in sda_list, or
 * NULL = width) into host arrays meta [num_parts][SDA_META_INTS] and num_splits [T+1]. For callers
 * that keep lengths on the host. A whole-token plan has no schedule: SDA_ERR_INVALID_ARG; the same
 * 2^31 bound on tile positions as sda_get_sched_meta. */
int sda_get_sched_meta_host(int T, int queries_per_len, const int32_t* lens /*host, nullable*/, int width,
                            const int32_t* extra_lens /*host, nullable*/, int extra_width /*0 = no extra list*/,
                            const sda_plan* plan /*host*/, int32_t* meta /*host*/, int32_t* num_splits /*host*/);

/* Decode attention (FlashMLA sparse_decode.h: sparse_attn_decode_interface; vLLM
 * swapab_decode_attn: __call__).
 *  q          bf16 [T][H][d_qk]; element (t, h, d) at q[t*q_stride_t + h*q_stride_h + d]; 16-byte
 *             aligned, strides multiples of 8 elements. Taken as given (no RoPE applied here).
 *  cache/list main cache and slot list; extra_cache/extra_list: both NULL or both set. The two
 *             caches may use different formats but must agree on d_qk.
 *  attn_sink  fp32 [H] or NULL: per-head logit in the units of scale * q.k; it adds exp(sink) to the
 *             softmax denominator and nothing to the numerator (vLLM swapab_decode_attn, step 9).
 *  scale      softmax scale applied to q.k (e.g. 1/sqrt(d_qk)).
 *  meta/num_splits  from sda_get_sched_meta with the same plan and lengths, or both NULL to have this
 *             call run the scheduler into the workspace first; both NULL for a whole-token plan
 *             (plan->whole_tokens), which runs neither the scheduler nor the combine.
 *  workspace  >= sda_workspace_bytes(T, H, d_v, plan) bytes, 256-byte aligned.
 *  out        bf16 [T][H][d_v]; element (t, h, d) at out[t*out_stride_t + h*out_stride_h + d],
 *             strides multiples of 8 elements, 16-byte aligned.
 *  lse        fp32 [T][H] at lse[t*lse_stride_t + h]: ln(exp(sink_h) + sum_i exp(z_i)); a token with
 *             no valid row gets out = 0 and lse = sink_h (-inf without a sink).
 * H in {16, 32, 64, 128}; (d_qk, d_v) in {(512, 512), (576, 512)}; 1 <= T; a split plan also needs
 * the scheduler's 2^31 bound on tile positions (sda_get_sched_meta), else SDA_ERR_UNSUPPORTED. */
int sda_sparse_decode_attn(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
                           const sda_cache* cache /*host*/, const sda_list* list /*host*/,
                           const sda_cache* extra_cache /*host, nullable*/, const sda_list* extra_list /*host, nullable*/,
                           const float* attn_sink, float scale, const sda_plan* plan /*host*/,
                           const int32_t* meta, const int32_t* num_splits, void* workspace, size_t workspace_bytes,
                           void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                           void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): sda_sparse_decode_attn without a workspace argument. The workspace is
 * a static device array of SDA_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends; this call allocates nothing. Every call on one GPU shares that GPU's array (no part of it
 * needs clearing: each call writes what it reads), so calls on one GPU whose streams overlap race and must
 * be ordered by the caller. A whole-token plan touches no workspace; a split plan needs
 * sda_noalloc_workspace_bytes(T, H, d_v, plan) <= SDA_SCRATCH_BYTES, else SDA_ERR_WORKSPACE. Other
 * arguments and errors as sda_sparse_decode_attn. */
#define SDA_SCRATCH_BYTES (64u << 20)

/* Host only. Scratch bytes sda_sparse_decode_attn_noalloc needs for this plan (0 for a whole-token plan). */
size_t sda_noalloc_workspace_bytes(int T, int H, int d_v, const sda_plan* plan /*host*/);

int sda_sparse_decode_attn_noalloc(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk,
                                   int d_v, const sda_cache* cache /*host*/, const sda_list* list /*host*/,
                                   const sda_cache* extra_cache /*host, nullable*/,
                                   const sda_list* extra_list /*host, nullable*/, const float* attn_sink, float scale,
                                   const sda_plan* plan /*host*/, const int32_t* meta, const int32_t* num_splits,
                                   void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse,
                                   int64_t lse_stride_t, void* stream);

/* The decode kernel alone (FlashMLA sparse_decode.h: impl->run, before the combine): same arguments
 * and checks as sda_sparse_decode_attn, but meta and num_splits are required (NULL for a whole-token
 * plan, whose tokens are all touched by a single workgroup, token t's partial going to split t) and
 * no combine runs.
 * Tokens touched by a single part get their final out/lse rows; the others get normalized fp32
 * partials in the workspace (o_accum at offset 0, lse_accum after it, as laid out by
 * sda_workspace_bytes) for a later sda_combine_splits. With out NULL (lse then unused) every token
 * leaves as a partial, as in the V4.1 call. */
int sda_decode_splits(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
                      const sda_cache* cache /*host*/, const sda_list* list /*host*/,
                      const sda_cache* extra_cache /*host, nullable*/, const sda_list* extra_list /*host, nullable*/,
                      const float* attn_sink, float scale, const sda_plan* plan /*host*/,
                      const int32_t* meta, const int32_t* num_splits, void* workspace, size_t workspace_bytes,
                      void* out, int64_t out_stride_t, int64_t out_stride_h, float* lse, int64_t lse_stride_t,
                      void* stream);

/* The V4.1 decode call (vLLM swapab_decode_attn: Q RoPE in stage_inputs; inverse RoPE and the MXFP8
 * output cast in device kernel step 9): q is taken before RoPE and the output leaves as fp8 with one
 * ue8m0 scale per 32 dims. RoPE covers dims [448, 512) as 32 GPT-J pairs (dims 448 + 2i, 449 + 2i),
 * rotated in fp32 (e' = fma(e, cos, -(o sin)), o' = fma(o, cos, e sin)) and rounded to bf16.
 *  positions     int64 [T], device: each token's position.
 *  cos_sin       fp32 [num_positions][cs_stride], device, 16-byte aligned: row p holds cos of pair i
 *                at [i] and its sin at [32 + i]; cs_stride >= 64 and a multiple of 4. A position
 *                outside [0, num_positions) rotates nothing (cos 1, sin 0).
 *  out_fp8       e4m3fn codes [T][H][512], code (t, h, d) at out_fp8[t*of_stride_t + h*of_stride_h + d];
 *                16-byte aligned, strides multiples of 16 bytes.
 *  out_scale     ue8m0 bytes [T][H][16], byte (t, h, c) at out_scale[t*os_stride_t + h*os_stride_h + c]
 *                for dims 32c .. 32c+31.
 * Per token and head, with x = the attention output in fp32 and its dims 448..511 rotated back per pair
 * (e' = fma(e, cos, sin o), o' = fma(o, cos, -(sin e))): per 32-dim chunk, amax = max(max |x|, 1e-10),
 * scale byte = the ue8m0 of amax * (1/448) rounded up to a power of two, codes = e4m3(x * 2^(127 - byte))
 * rounded to nearest even. */
typedef struct sda_v41 {
  const int64_t* positions;
  const float* cos_sin;
  int64_t cs_stride;
  int64_t num_positions;
  uint8_t* out_fp8;
  int64_t of_stride_t, of_stride_h;
  uint8_t* out_scale;
  int64_t os_stride_t, os_stride_h;
} sda_v41;

/* Host only. Workspace of sda_sparse_decode_attn_v41: that of sda_workspace_bytes(T, H, 512, plan)
 * plus the rotated query dims 448..511 (bf16 [T][H][64]). */
size_t sda_workspace_bytes_v41(int T, int H, const sda_plan* plan /*host*/);

/* V4.1 decode: the arguments of sda_sparse_decode_attn with d_qk = d_v = 512, the bf16 output replaced
 * by `v41` (host descriptor, device buffers) and lse optional (NULL: not written). Every token passes
 * through the combine, where the output cast happens (with a whole-token plan: no scheduler, and the
 * combine takes token t's single partial from split t). Errors as sda_sparse_decode_attn, plus
 * SDA_ERR_INVALID_ARG for a bad v41 descriptor. */
int sda_sparse_decode_attn_v41(const void* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H,
                               const sda_cache* cache /*host*/, const sda_list* list /*host*/,
                               const sda_cache* extra_cache /*host, nullable*/,
                               const sda_list* extra_list /*host, nullable*/, const float* attn_sink, float scale,
                               const sda_plan* plan /*host*/, const int32_t* meta, const int32_t* num_splits,
                               void* workspace, size_t workspace_bytes, const sda_v41* v41 /*host*/,
                               float* lse /*nullable*/, int64_t lse_stride_t, void* stream);

/* Host only. Byte offsets of lse_accum in the workspace of this plan (o_accum starts at 0). */
size_t sda_workspace_lse_offset(int T, int H, int d_v, const sda_plan* plan /*host*/);

/* LSE merge of split partials (FlashMLA sparse_decode.h: run_flash_mla_combine_kernel; the merge of
 * vLLM swapab_decode_attn step 9 with the sink folded in once). For every token t with
 * n_t = num_splits[t+1] - num_splits[t] >= 2: with s = num_splits[t] + k for k < n_t,
 *   M = max(sink_h, lse_accum[s][h]), den = exp(sink_h - M) + sum_k exp(lse_accum[s][h] - M),
 *   out = sum_k exp(lse_accum[s][h] - M) * o_accum[s][h][:] / den,  lse = M + ln(den).
 * o_accum [*][H][d_v] fp32 holds normalized partials; a part with no rows has lse -inf. Tokens with
 * n_t < 2 are left untouched (the decode kernel writes them directly). H in {16, 32, 64, 128}, d_v = 512;
 * o_accum and out 16-byte aligned, out strides multiples of 8 elements. */
int sda_combine_splits(int T, int H, int d_v, const float* o_accum, const float* lse_accum,
                       const int32_t* num_splits, const float* attn_sink, void* out, int64_t out_stride_t,
                       int64_t out_stride_h, float* lse, int64_t lse_stride_t, void* stream);

/* Host only. Static description of a status code. */
const char* sda_status_string(int status);

/* Host only. Message of the last SDA_ERR_HIP (or argument error) on the calling thread. */
const char* sda_last_error(void);

/* Host only. Record bytes and d_qk of a format (-1 if unknown). */
int sda_record_bytes(int format);
int sda_format_dims(int format);

#ifdef __cplusplus
}
#endif
#endif
