/* oracle.c -- plain fp64 CPU reference for paged, quantized, shared-KV decode
 * attention. TEST INFRASTRUCTURE ONLY (see oracle.h): the library under test
 * never loads it.
 *
 * Two passes per (token, head): scores and their max, then exponentials, the
 * weighted sum and the log-sum-exp. Everything is double precision; there is
 * no blocking, no online rescaling and no splitting.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- decoders */

/* e4m3fn (OCP 8-bit floating point, "E4M3"): 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6); the
 * all-ones exponent is a normal binade except S.1111.111, which is NaN. */
double orc_e4m3(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* e2m1 (OCP MX, FP4): 1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * exponent field 0 is subnormal (m * 0.5). No NaN or infinity. */
double orc_e2m1(int nibble) {
  int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* ue8m0 (OCP MX scale, "E8M0"): an unsigned biased exponent, 2^(byte - 127),
 * no sign and no mantissa; 0xFF is NaN. */
double orc_ue8m0(int byte) {
  byte &= 0xFF;
  if (byte == 0xFF) return NAN;
  return ldexp(1.0, byte - 127);
}

/* bf16 is the upper half of an IEEE binary32 word. */
double orc_bf16(int bits) {
  uint32_t u = ((uint32_t)bits & 0xFFFFu) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double f32_le(const uint8_t* p) {
  uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int orc_record_bytes(int format) {
  switch (format) {
    case ORC_FP8_SLOTSCALE: return 512;
    case ORC_FP8_528: return 512 + 4 * 4;       /* codes, then one fp32 per 128 dims       */
    case ORC_NVFP4_288: return 256 + 32;        /* packed e2m1, then one e4m3 per 16 dims  */
    case ORC_V32_656: return 512 + 4 * 4 + 64 * 2; /* codes, 4 fp32 scales, 64 bf16 dims   */
    case ORC_FP8_UE8M0: return 512 + 16;        /* codes, then one ue8m0 per 32 dims       */
    case ORC_MODEL1_584: return 448 + 64 * 2 + 448 / 64 + 1; /* codes, 64 bf16 dims, 7 ue8m0, pad */
    default: return -1;
  }
}

int orc_record_dims(int format) {
  switch (format) {
    case ORC_FP8_SLOTSCALE:
    case ORC_FP8_528:
    case ORC_NVFP4_288:
    case ORC_FP8_UE8M0:
    case ORC_MODEL1_584: return 512;
    case ORC_V32_656: return 576;
    default: return -1;
  }
}

/* Slot addressing of the paged cache (vLLM swapab_decode_attn page, stage_inputs:
 * page = sid / page_size, offset = sid mod page_size, record at
 * base + page*page_stride + offset*record; slot ids outside [0, slots) are
 * masked). Dequantization multiplies each code by its stored scale. */
int orc_decode_slot(const orc_cache* c, int64_t sid, double* k) {
  int64_t slots = c->num_pages * (int64_t)c->page_size;
  if (sid < 0 || sid >= slots) return 0;
  int rec = orc_record_bytes(c->format);
  int64_t page = sid / c->page_size, off = sid % c->page_size;
  const uint8_t* r = c->base + page * c->page_stride + off * (int64_t)rec;
  int d;
  switch (c->format) {
    case ORC_FP8_SLOTSCALE: {
      double s = (double)c->slot_scale[sid];
      for (d = 0; d < 512; d++) k[d] = orc_e4m3(r[d]) * s;
      break;
    }
    case ORC_FP8_528:
    case ORC_V32_656: {
      for (d = 0; d < 512; d++) k[d] = orc_e4m3(r[d]) * f32_le(r + 512 + 4 * (d / 128));
      if (c->format == ORC_V32_656)
        for (d = 0; d < 64; d++) k[512 + d] = orc_bf16(r[528 + 2 * d] | (r[528 + 2 * d + 1] << 8));
      break;
    }
    case ORC_FP8_UE8M0: {
      /* vLLM swapab_decode_attn page, stage_inputs (fp8 branch): 16-byte chunk c
       * holds dims 16c..16c+15 and takes scale byte c / 2, i.e. scale byte g
       * covers dims 32g..32g+31 */
      for (d = 0; d < 512; d++) k[d] = orc_e4m3(r[d]) * orc_ue8m0(r[512 + d / 32]);
      break;
    }
    case ORC_MODEL1_584: {
      /* FlashMLA sparse_decode.h, MODEL1 bytes_per_token: 448 e4m3 codes, 64 bf16
       * dims, one ue8m0 scale per 64 coded dims, one pad byte. The page gives the
       * parts and the total only; they are taken in the order its sum lists them:
       * bytes [0,448) codes of dims 0..447, [448,576) dims 448..511 as bf16,
       * [576,583) scale byte g for dims 64g..64g+63, byte 583 unused. */
      for (d = 0; d < 448; d++) k[d] = orc_e4m3(r[d]) * orc_ue8m0(r[576 + d / 64]);
      for (d = 0; d < 64; d++) k[448 + d] = orc_bf16(r[448 + 2 * d] | (r[448 + 2 * d + 1] << 8));
      break;
    }
    case ORC_NVFP4_288: {
      for (d = 0; d < 512; d++) {
        int byte = r[d / 2];
        int nib = (d % 2 == 0) ? (byte & 15) : (byte >> 4);   /* low nibble = even element */
        k[d] = orc_e2m1(nib) * orc_e4m3(r[256 + d / 16]);
      }
      break;
    }
    default: return 0;
  }
  return 1;
}

/* ---------------------------------------------------------------- attention */

typedef struct {
  const uint16_t* q;
  int64_t qst, qsh;
  int T, H, d_qk, d_v;
  const orc_cache* c[2];
  const orc_list* l[2];
  int nl;
  const float* sink;
  float scale;
  double* out;
  double* lse;
  double* out_abs;  /* optional: sum_i w_i |v_i| / den, with the weights of out */
  int t_begin, t_step;
} job_t;

/* Rows of token t: list entries j < clamp(lens[t], 0, width) whose slot decodes. */
static int gather_token(const job_t* jb, int t, double* rows, int max_rows) {
  int n = 0, li, j;
  for (li = 0; li < jb->nl; li++) {
    const orc_list* L = jb->l[li];
    int len = L->lens ? L->lens[t] : L->width;
    if (len < 0) len = 0;
    if (len > L->width) len = L->width;
    for (j = 0; j < len && n < max_rows; j++) {
      int32_t sid = L->idx[(int64_t)t * L->row_stride + j];
      if (orc_decode_slot(jb->c[li], sid, rows + (int64_t)n * jb->d_qk)) n++;
    }
  }
  return n;
}

static void token_heads(const job_t* jb, int t, const double* rows, int n, double* z, double* qd) {
  int h, i, d;
  for (h = 0; h < jb->H; h++) {
    double* o = jb->out + ((int64_t)t * jb->H + h) * jb->d_v;
    double* oa = jb->out_abs ? jb->out_abs + ((int64_t)t * jb->H + h) * jb->d_v : NULL;
    double* lse = jb->lse + (int64_t)t * jb->H + h;
    int has_sink = jb->sink != NULL;
    double sk = has_sink ? (double)jb->sink[h] : -INFINITY;
    for (d = 0; d < jb->d_v; d++) o[d] = 0.0;
    if (oa)
      for (d = 0; d < jb->d_v; d++) oa[d] = 0.0;
    for (d = 0; d < jb->d_qk; d++) qd[d] = orc_bf16(jb->q[(int64_t)t * jb->qst + (int64_t)h * jb->qsh + d]);
    if (n == 0) {            /* no rows: zero output; the sink alone is the log-sum-exp */
      *lse = has_sink ? sk : -INFINITY;
      continue;
    }
    if (sk == INFINITY) {    /* an infinite sink takes all the probability mass        */
      *lse = INFINITY;
      continue;
    }
    double M = sk;
    for (i = 0; i < n; i++) {
      const double* k = rows + (int64_t)i * jb->d_qk;
      double acc = 0.0;
      for (d = 0; d < jb->d_qk; d++) acc += qd[d] * k[d];
      z[i] = (double)jb->scale * acc;
      if (z[i] > M) M = z[i];
    }
    double den = has_sink ? exp(sk - M) : 0.0;
    for (i = 0; i < n; i++) {
      double w = exp(z[i] - M);
      const double* v = rows + (int64_t)i * jb->d_qk;
      den += w;
      for (d = 0; d < jb->d_v; d++) o[d] += w * v[d];
      if (oa)
        for (d = 0; d < jb->d_v; d++) oa[d] += w * fabs(v[d]);
    }
    for (d = 0; d < jb->d_v; d++) o[d] /= den;
    if (oa)
      for (d = 0; d < jb->d_v; d++) oa[d] /= den;
    *lse = M + log(den);
  }
}

static void* run_job(void* arg) {
  const job_t* jb = (const job_t*)arg;
  int max_rows = 0, li, t;
  for (li = 0; li < jb->nl; li++) max_rows += jb->l[li]->width;
  double* rows = (double*)malloc(sizeof(double) * (size_t)(max_rows > 0 ? max_rows : 1) * jb->d_qk);
  double* z = (double*)malloc(sizeof(double) * (size_t)(max_rows > 0 ? max_rows : 1));
  double* qd = (double*)malloc(sizeof(double) * (size_t)jb->d_qk);
  for (t = jb->t_begin; t < jb->T; t += jb->t_step) {
    int n = gather_token(jb, t, rows, max_rows);
    token_heads(jb, t, rows, n, z, qd);
  }
  free(rows);
  free(z);
  free(qd);
  return NULL;
}

int orc_attn(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
             const orc_cache* cache, const orc_list* list, const orc_cache* xcache, const orc_list* xlist,
             const float* sink, float scale, double* out, double* lse, int nthreads) {
  return orc_attn_abs(q, q_stride_t, q_stride_h, T, H, d_qk, d_v, cache, list, xcache, xlist, sink, scale, out, lse,
                      NULL, nthreads);
}

int orc_attn_abs(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H, int d_qk, int d_v,
                 const orc_cache* cache, const orc_list* list, const orc_cache* xcache, const orc_list* xlist,
                 const float* sink, float scale, double* out, double* lse, double* out_abs, int nthreads) {
  if (!q || !cache || !list || !out || !lse || T < 0 || H <= 0) return -1;
  if ((xcache == NULL) != (xlist == NULL)) return -1;
  if (orc_record_dims(cache->format) != d_qk) return -1;
  if (xcache && orc_record_dims(xcache->format) != d_qk) return -1;
  if (d_v > d_qk || d_v <= 0) return -1;
  job_t base;
  memset(&base, 0, sizeof(base));
  base.q = q; base.qst = q_stride_t; base.qsh = q_stride_h;
  base.T = T; base.H = H; base.d_qk = d_qk; base.d_v = d_v;
  base.c[0] = cache; base.l[0] = list; base.nl = 1;
  if (xcache) { base.c[1] = xcache; base.l[1] = xlist; base.nl = 2; }
  base.sink = sink; base.scale = scale; base.out = out; base.lse = lse; base.out_abs = out_abs;
  if (nthreads <= 1 || T <= 1) {
    base.t_begin = 0; base.t_step = 1;
    run_job(&base);
    return 0;
  }
  if (nthreads > T) nthreads = T;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  job_t* jobs = (job_t*)malloc(sizeof(job_t) * (size_t)nthreads);
  int i;
  for (i = 0; i < nthreads; i++) {
    jobs[i] = base;
    jobs[i].t_begin = i;
    jobs[i].t_step = nthreads;
    pthread_create(&th[i], NULL, run_job, &jobs[i]);
  }
  for (i = 0; i < nthreads; i++) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return 0;
}

/* LSE merge of normalized partials (dsv4 production.py, _run_fmha_segmented:
 * O = sum_i e^{lse_i} O_i / sum_i e^{lse_i}, here shifted by the max for range;
 * the sink is one more term of the denominator, folded in once, as in the
 * vLLM swapab_decode_attn merge). */
void orc_merge(int n, int H, int d_v, const double* o, const double* part_lse, const float* sink,
               double* out, double* lse) {
  int h, i, d;
  for (h = 0; h < H; h++) {
    double sk = sink ? (double)sink[h] : -INFINITY;
    double M = sk;
    double* oh = out + (int64_t)h * d_v;
    for (d = 0; d < d_v; d++) oh[d] = 0.0;
    for (i = 0; i < n; i++) {
      double li = part_lse[(int64_t)i * H + h];
      if (li > M) M = li;
    }
    if (M == -INFINITY) { lse[h] = -INFINITY; continue; }
    if (M == INFINITY) { lse[h] = INFINITY; continue; }
    double den = sink ? exp(sk - M) : 0.0;
    for (i = 0; i < n; i++) {
      double li = part_lse[(int64_t)i * H + h];
      if (li == -INFINITY) continue;
      double w = exp(li - M);
      den += w;
      const double* oi = o + ((int64_t)i * H + h) * d_v;
      for (d = 0; d < d_v; d++) oh[d] += w * oi[d];
    }
    for (d = 0; d < d_v; d++) oh[d] /= den;
    lse[h] = M + log(den);
  }
}

/* ------------------------------------------------- V4.1 prologue / epilogue */

#define ORC_ROPE_START 448
#define ORC_ROPE_PAIRS 32

static float f32_of_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round to nearest even on the 16 dropped bits: add 0x7FFF plus the lowest kept
 * bit, then truncate (a carry into the exponent is the correct rounding up). */
int orc_bf16_rne(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (int)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (int)(u >> 16);
}

/* e4m3fn values are m/8 * 2^-6 (subnormal, code m) and (1 + m/8) * 2^(e-7)
 * (code 8e + m); the codes of non-negative values are monotone in the value,
 * so rounding the value to the nearest multiple of its binade's step and
 * counting steps gives the code. */
int orc_e4m3_encode(float x) {
  if (isnan(x)) return 0x7F;
  int sign = signbit(x) ? 0x80 : 0;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  int code;
  if (a < ldexp(1.0, -6)) {
    code = (int)nearbyint(ldexp(a, 9));          /* steps of 2^-9; 8 steps is the first normal */
  } else {
    int e;
    frexp(a, &e);                                /* a = f * 2^e, f in [0.5, 1)                   */
    int be = e - 1;                              /* a in [2^be, 2^(be+1))                        */
    int m = (int)nearbyint(ldexp(a, 3 - be)) - 8; /* eighths above 1; 8 carries into the binade  */
    code = 8 * (be + 7) + m;
  }
  if (code > 0x7E) code = 0x7E;
  return sign | code;
}

static void cos_sin_of(const float* cs, int64_t stride, int64_t npos, int64_t pos, int i, float* c, float* s) {
  if (pos < 0 || pos >= npos) {
    *c = 1.0f;
    *s = 0.0f;
    return;
  }
  *c = cs[pos * stride + i];
  *s = cs[pos * stride + ORC_ROPE_PAIRS + i];
}

void orc_rope_q(const uint16_t* q, int64_t q_stride_t, int64_t q_stride_h, int T, int H,
                const int64_t* positions, const float* cos_sin, int64_t cs_stride, int64_t num_positions,
                uint16_t* q_out) {
  int t, h, d, i;
  for (t = 0; t < T; t++) {
    for (h = 0; h < H; h++) {
      const uint16_t* src = q + (int64_t)t * q_stride_t + (int64_t)h * q_stride_h;
      uint16_t* dst = q_out + ((int64_t)t * H + h) * 512;
      for (d = 0; d < 512; d++) dst[d] = src[d];
      for (i = 0; i < ORC_ROPE_PAIRS; i++) {
        float c, s;
        cos_sin_of(cos_sin, cs_stride, num_positions, positions[t], i, &c, &s);
        int e = ORC_ROPE_START + 2 * i;
        float qe = f32_of_bf16(src[e]), qo = f32_of_bf16(src[e + 1]);
        float re = fmaf(qe, c, -(qo * s));
        float ro = fmaf(qo, c, qe * s);
        dst[e] = (uint16_t)orc_bf16_rne(re);
        dst[e + 1] = (uint16_t)orc_bf16_rne(ro);
      }
    }
  }
}

/* ue8m0 of y rounded up to a power of two: the biased exponent, plus one when
 * any mantissa bit is set (y normal and positive here). */
static int ue8m0_round_up(float y) {
  uint32_t u;
  memcpy(&u, &y, 4);
  int e = (int)((u >> 23) & 0xFFu);
  return e + ((u & 0x7FFFFFu) != 0u ? 1 : 0);
}

void orc_mxfp8_out(const double* out, int T, int H, const int64_t* positions, const float* cos_sin,
                   int64_t cs_stride, int64_t num_positions, uint8_t* codes, uint8_t* scales) {
  int t, h, d, i, k;
  float x[512];
  for (t = 0; t < T; t++) {
    for (h = 0; h < H; h++) {
      const double* o = out + ((int64_t)t * H + h) * 512;
      for (d = 0; d < 512; d++) x[d] = (float)o[d];
      for (i = 0; i < ORC_ROPE_PAIRS; i++) {
        float c, s;
        cos_sin_of(cos_sin, cs_stride, num_positions, positions[t], i, &c, &s);
        int e = ORC_ROPE_START + 2 * i;
        float oe = x[e], oo = x[e + 1];
        x[e] = fmaf(oe, c, s * oo);
        x[e + 1] = fmaf(oo, c, -(s * oe));
      }
      uint8_t* cd = codes + ((int64_t)t * H + h) * 512;
      uint8_t* sc = scales + ((int64_t)t * H + h) * 16;
      for (k = 0; k < 16; k++) {
        float amax = 0.0f;
        for (d = 32 * k; d < 32 * k + 32; d++) amax = fmaxf(amax, fabsf(x[d]));
        amax = fmaxf(amax, 1e-10f);
        int ex = ue8m0_round_up(amax * (float)(1.0 / 448.0));
        uint32_t ib = (uint32_t)(254 - ex) << 23;
        float inv;
        memcpy(&inv, &ib, 4);
        sc[k] = (uint8_t)ex;
        for (d = 32 * k; d < 32 * k + 32; d++) cd[d] = (uint8_t)orc_e4m3_encode(x[d] * inv);
      }
    }
  }
}
