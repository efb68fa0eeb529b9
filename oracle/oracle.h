/* oracle.h -- plain fp64 CPU reference for single-step decode attention over a
 * paged, quantized, shared-KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's CPU
 * baseline may load this code; the library under test never does, and the two
 * share no source, header, table or helper.
 *
 * What it computes (plain definition, no online softmax, no splitting): for
 * each token t and head h, over the multiset R_t of valid rows of the main list
 * followed by the extra list,
 *     z_i = scale * sum_d q[t,h,d] * k_i[d]
 *     M   = max(max_i z_i, sink_h)              (sink term only when a sink is given)
 *     den = sum_i exp(z_i - M) + exp(sink_h - M)
 *     out = sum_i exp(z_i - M) * v_i / den,   v_i = k_i[0:d_v]
 *     lse = M + ln(den)
 * An empty R_t gives out = 0 and lse = sink_h (or -inf without a sink).
 * Sources: masked MQA softmax attention of native_swa_decode.py
 * (_fallback_batched_sdp), the gather/validity rules of vLLM's
 * swapab_decode_attn (stage_inputs), the sink merge of the same page (device
 * kernel step 9) and the split/LSE merge of dsv4 production.py
 * (_run_fmha_segmented).
 */
#ifndef SDA_ORACLE_H
#define SDA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FP8_SLOTSCALE = 0, ORC_FP8_528 = 1, ORC_NVFP4_288 = 2, ORC_V32_656 = 3, ORC_FP8_UE8M0 = 4,
       ORC_MODEL1_584 = 5 };

typedef struct {
  const uint8_t* base;     /* host bytes of page 0                                   */
  int64_t num_pages;
  int32_t page_size;       /* slots per page                                          */
  int64_t page_stride;     /* bytes between consecutive pages                         */
  int32_t format;          /* ORC_*                                                   */
  const float* slot_scale; /* [num_pages*page_size], ORC_FP8_SLOTSCALE only           */
} orc_cache;

typedef struct {
  const int32_t* idx;      /* [T][row_stride] slot ids, -1 = none                     */
  int64_t row_stride;
  int32_t width;
  const int32_t* lens;     /* [T] or NULL (= width)                                   */
} orc_list;

/* Scalar decoders (OCP 8-bit floating point and MX specifications). */
double orc_e4m3(int code);          /* e4m3fn; 0x7F / 0xFF are NaN                          */
double orc_e2m1(int nibble);        /* e2m1                                                */
double orc_bf16(int bits);          /* bf16 bit pattern                                    */
double orc_ue8m0(int byte);         /* 2^(byte - 127); 0xFF is NaN                         */
int orc_record_bytes(int format);   /* 512, 528, 288, 656, 528, 584; -1 if unknown         */
int orc_record_dims(int format);    /* d_qk of the format: 512 or 576                      */

/* Decode slot `sid` into k[0..dims). Returns 1 if the slot is in range and was
 * decoded, 0 if it is masked (sid < 0 or sid >= num_pages*page_size). */
int orc_decode_slot(const orc_cache* c, int64_t sid, double* k);

/* Full attention. q: bf16 bits, element (t,h,d) at q[t*q_stride_t + h*q_stride_h + d].
 * extra cache/list may be NULL together. sink: [H] or NULL. out: [T][H][d_v], lse: [T][H].
 * Returns 0, or -1 on inconsistent arguments. nthreads <= 1 runs on the caller's thread. */
int orc_attn(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
             const orc_cache* cache, const orc_list* list, const orc_cache* xcache, const orc_list* xlist,
             const float* sink, float scale, double* out, double* lse, int nthreads);

/* orc_attn plus out_abs [T][H][d_v] (nullable): sum_i exp(z_i - M) |v_i| / den, the weighted mean of the
 * rows' magnitudes under the same weights (zero for an empty token). It is the scale that a relative error
 * in the weights moves the output by (|sum_i w_i d_i v_i| <= max |d_i| out_abs), which the tests' rounding
 * tolerance is stated in; it is no part of the method. */
int orc_attn_abs(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
                 const orc_cache* cache, const orc_list* list, const orc_cache* xcache, const orc_list* xlist,
                 const float* sink, float scale, double* out, double* lse, double* out_abs, int nthreads);

/* ---- V4.1 decode prologue and epilogue (vLLM swapab_decode_attn page: Q RoPE
 * in stage_inputs, inverse RoPE and the MXFP8 output cast in device kernel step
 * 9). Both follow the page's single-precision steps, so that the quantized
 * results are decided in the precision the page takes them in.
 * RoPE covers dims [448, 512) as 32 GPT-J pairs (dims 448 + 2i, 449 + 2i);
 * cos_sin row p holds cos of pair i at [i] and its sin at [32 + i]. A position
 * outside [0, num_positions) rotates nothing (cos 1, sin 0). */

/* fp32 -> bf16 bits, round to nearest even (NaN stays NaN). */
int orc_bf16_rne(float x);
/* fp32 -> e4m3fn code, round to nearest even, saturating at +-448 (NaN -> 0x7F). */
int orc_e4m3_encode(float x);
/* q_out[t][h][d] (bf16 bits, [T][H][512] contiguous): q with its dims 448..511
 * rotated by the angle of positions[t]: per pair, in fp32,
 *   e' = fma(e, cos, -(o * sin)),  o' = fma(o, cos, e * sin),  rounded to bf16. */
void orc_rope_q(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H,
                const int64_t* positions, const float* cos_sin, int64_t cs_stride, int64_t num_positions,
                uint16_t* q_out);
/* MXFP8 output of attention results out [T][H][512] (taken to fp32 first): dims
 * 448..511 rotated back per pair (e' = fma(e, cos, sin * o), o' = fma(o, cos,
 * -(sin * e))), then per 32-dim chunk: amax = max(max |x|, 1e-10), scale byte =
 * the ue8m0 of amax * (1/448) rounded up to a power of two, codes =
 * e4m3(x * 2^(127 - byte)). codes: [T][H][512], scales: [T][H][16]. */
void orc_mxfp8_out(const double* out, int T, int H, const int64_t* positions, const float* cos_sin,
                   int64_t cs_stride, int64_t num_positions, uint8_t* codes, uint8_t* scales);

/* LSE merge of n normalized partial results of one (token, head) group:
 * o: [n][H][d_v], part_lse: [n][H] (a part with no rows has lse -inf and is ignored).
 * The sink (may be NULL) enters the denominator once. out: [H][d_v], lse: [H]. */
void orc_merge(int n, int H, int d_v, const double* o, const double* part_lse, const float* sink,
               double* out, double* lse);

#ifdef __cplusplus
}
#endif
#endif
