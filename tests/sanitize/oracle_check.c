/* Drives every oracle entry point over small inputs of every record format, the edge cases included
 * (slot -1 and out of range, lengths < 0 and > width, empty tokens, sinks of +-inf, the extra list,
 * several threads, positions outside the RoPE table), for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer. Exits 0 when every call returns and the results are sane. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) {
  rng_state = rng_state * 1664525u + 1013904223u;
  return rng_state >> 8;
}

static int check_format(int fmt, int nthreads) {
  const int rec = orc_record_bytes(fmt), dims = orc_record_dims(fmt);
  const int page = 8, pages = 4, slots = page * pages, T = 5, H = 3, W = 12, XW = 7;
  const int64_t stride = (int64_t)page * rec + 16;
  uint8_t* data = (uint8_t*)malloc((size_t)pages * stride);
  for (int64_t i = 0; i < pages * stride; ++i) data[i] = (uint8_t)(rnd() & 0x77);  /* no NaN codes */
  for (int s = 0; s < slots; ++s) {  /* scales: fp32 1.0, or ue8m0 bytes 120..134 */
    uint8_t* r = data + (s / page) * stride + (s % page) * rec;
    if (fmt == ORC_FP8_528 || fmt == ORC_V32_656) {
      const float one = 1.0f;
      for (int g = 0; g < 4; ++g) memcpy(r + 512 + 4 * g, &one, 4);
    }
    if (fmt == ORC_FP8_UE8M0)
      for (int g = 0; g < 16; ++g) r[512 + g] = (uint8_t)(120 + rnd() % 15);
    if (fmt == ORC_MODEL1_584)
      for (int g = 0; g < 7; ++g) r[576 + g] = (uint8_t)(120 + rnd() % 15);
  }
  float* ss = NULL;
  if (fmt == ORC_FP8_SLOTSCALE) {
    ss = (float*)malloc(sizeof(float) * slots);
    for (int s = 0; s < slots; ++s) ss[s] = 0.5f + (float)(rnd() % 100) / 100.0f;
  }
  orc_cache c = {data, pages, page, stride, fmt, ss};
  int32_t idx[5 * 12], xidx[5 * 7], lens[5] = {0, 3, 12, -4, 40}, xlens[5] = {7, 0, 2, 9, 1};
  for (int i = 0; i < T * W; ++i) idx[i] = (int32_t)(rnd() % (slots + 6)) - 3;  /* -3 .. slots + 2 */
  for (int i = 0; i < T * XW; ++i) xidx[i] = (int32_t)(rnd() % slots);
  orc_list L = {idx, W, W, lens}, X = {xidx, XW, XW, xlens};
  uint16_t* q = (uint16_t*)malloc(sizeof(uint16_t) * T * H * dims);
  for (int i = 0; i < T * H * dims; ++i) q[i] = (uint16_t)(0x3C00 + (rnd() & 0x3FF)) ^ (uint16_t)((rnd() & 1) << 15);
  const float sink[3] = {0.5f, -INFINITY, 2.0f};
  double *out = (double*)malloc(sizeof(double) * T * H * 512), *oabs = (double*)malloc(sizeof(double) * T * H * 512);
  double lse[15];
  int bad = 0;
  if (orc_attn_abs(q, (int64_t)H * dims, dims, T, H, dims, 512, &c, &L, &c, &X, sink, 0.05f, out, lse, oabs,
                   nthreads) != 0)
    ++bad;
  for (int i = 0; i < T * H * 512; ++i)
    if (!isfinite(out[i]) || !(oabs[i] >= fabs(out[i]) * (1 - 1e-12))) ++bad;
  if (orc_attn(q, (int64_t)H * dims, dims, T, H, dims, 512, &c, &L, NULL, NULL, NULL, 0.05f, out, lse, 1) != 0) ++bad;
  if (!(isinf(lse[0]) && lse[0] < 0)) ++bad;  /* token 0 has no rows and no sink */
  double k[576];
  for (int s = -2; s < slots + 2; ++s) orc_decode_slot(&c, s, k);
  free(data); free(ss); free(q); free(out); free(oabs);
  return bad;
}

int main(void) {
  int bad = 0;
  for (int code = 0; code < 256; ++code) { (void)orc_e4m3(code); (void)orc_ue8m0(code); }
  for (int nib = 0; nib < 16; ++nib) (void)orc_e2m1(nib);
  for (int b = 0; b < 65536; b += 7) (void)orc_bf16(b);
  const int fmts[6] = {ORC_FP8_SLOTSCALE, ORC_FP8_528, ORC_NVFP4_288, ORC_V32_656, ORC_FP8_UE8M0, ORC_MODEL1_584};
  for (int i = 0; i < 6; ++i) bad += check_format(fmts[i], 1 + (i % 3));
  /* merge: a part with no rows, a sink of +inf */
  double o[3 * 2 * 512], pl[3 * 2] = {0.5, -INFINITY, 1.0, 2.0, -INFINITY, -INFINITY}, mo[2 * 512], ml[2];
  for (int i = 0; i < 3 * 2 * 512; ++i) o[i] = (double)(rnd() % 100) / 50.0 - 1.0;
  const float sk[2] = {INFINITY, -1.0f};
  orc_merge(3, 2, 512, o, pl, sk, mo, ml);
  orc_merge(3, 2, 512, o, pl, NULL, mo, ml);
  /* RoPE and the MXFP8 cast, positions inside and outside the table */
  uint16_t qq[2 * 2 * 512], qo[2 * 2 * 512];
  for (int i = 0; i < 2 * 2 * 512; ++i) qq[i] = (uint16_t)(0x3F00 + (rnd() & 0xFF));
  float cs[4 * 64];
  for (int i = 0; i < 4 * 64; ++i) cs[i] = (float)(rnd() % 200) / 100.0f - 1.0f;
  const int64_t pos[2] = {3, 9};
  orc_rope_q(qq, 1024, 512, 2, 2, pos, cs, 64, 4, qo);
  double ao[2 * 2 * 512];
  for (int i = 0; i < 2 * 2 * 512; ++i) ao[i] = (double)(rnd() % 1000) / 10.0 - 50.0;
  ao[0] = 1e30; ao[1] = 0.0;
  uint8_t codes[2 * 2 * 512], sc[2 * 2 * 16];
  orc_mxfp8_out(ao, 2, 2, pos, cs, 64, 4, codes, sc);
  for (int i = 0; i < 100; ++i) { (void)orc_bf16_rne((float)i * 1.37f - 50.0f); (void)orc_e4m3_encode((float)i * 9.1f - 400.0f); }
  (void)orc_e4m3_encode(NAN);
  printf("oracle sanitizer check: %s\n", bad ? "FAILED" : "ok");
  return bad ? 1 : 0;
}
