/* Drives every entry point of the CPU oracle on small inputs, for runs under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitize.py).
 * Exits non-zero if a result is not finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hkv_oracle.h"

static uint64_t st = 12345;
static float rnd(void) {
  const uint64_t z = orc_splitmix64_next(&st);
  return (float)((double)(z >> 11) * 0x1.0p-53 * 4.0 - 2.0);
}

static int run_format(const char* dtype, int32_t d, int32_t rope) {
  orc_format f;
  if (orc_format_init(&f, dtype, d, rope) != ORC_OK) return 1;
  const int64_t T = 37;
  const int32_t H = 2, HQ = 4, PS = 16;
  const int32_t pages = (int32_t)((T + PS - 1) / PS);
  float* k = malloc(sizeof(float) * T * H * d);
  float* v = malloc(sizeof(float) * T * H * d);
  for (int64_t i = 0; i < T * H * d; ++i) {
    k[i] = rnd();
    v[i] = rnd();
  }
  for (int32_t i = 0; i < d; ++i) k[i] = 0.0f; /* an all-zero head vector */
  uint8_t* slots = malloc((size_t)(T * H * f.slot_bytes));
  orc_quantize(&f, k, v, T, H, slots);
  float* kd = malloc(sizeof(float) * T * H * d);
  float* vd = malloc(sizeof(float) * T * H * d);
  double* kd64 = malloc(sizeof(double) * T * H * d);
  double* vd64 = malloc(sizeof(double) * T * H * d);
  orc_dequantize(&f, slots, T, H, 0, kd, vd);
  orc_dequantize(&f, slots, T, H, 1, kd, vd);
  orc_dequantize_f64(&f, slots, T, H, kd64, vd64);
  /* paged cache: identity page table */
  uint8_t* cache = calloc((size_t)pages * H * PS * f.slot_bytes, 1);
  for (int64_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < H; ++h)
      memcpy(cache + (((t / PS) * H + h) * PS + t % PS) * f.slot_bytes,
             slots + (t * H + h) * f.slot_bytes, (size_t)f.slot_bytes);
  int32_t bt[8];
  for (int32_t p = 0; p < 8; ++p) bt[p] = p < pages ? p : 0;
  const int32_t nq = 3;
  int32_t q_to_req[3] = {0, 0, 0}, q_to_klen[3] = {(int32_t)T, 1, 0};
  float* q = malloc(sizeof(float) * nq * HQ * d);
  for (int32_t i = 0; i < nq * HQ * d; ++i) q[i] = rnd();
  double* out = malloc(sizeof(double) * nq * HQ * d);
  orc_attention(&f, q, nq, HQ, cache, H, PS, bt, 8, q_to_req, q_to_klen, 1.0 / sqrt((double)d), out);
  int bad = 0;
  for (int32_t i = 0; i < nq * HQ * d; ++i) bad |= !isfinite(out[i]);
  double lse[3 * HQ];
  orc_attention_lse(&f, q, nq, HQ, cache, H, PS, bt, 8, q_to_req, q_to_klen,
                    1.0 / sqrt((double)d), out, lse);
  for (int32_t i = 0; i < nq * HQ * d; ++i) bad |= !isfinite(out[i]);
  for (int32_t i = 0; i < 2 * HQ; ++i) bad |= !isfinite(lse[i]); /* klen T and 1 */
  for (int32_t i = 2 * HQ; i < 3 * HQ; ++i) bad |= !(isinf(lse[i]) && lse[i] < 0); /* klen 0 */
  for (int64_t i = 0; i < T * H * d; ++i) bad |= !isfinite(kd[i]) || !isfinite(vd64[i]);
  free(k), free(v), free(slots), free(kd), free(vd), free(kd64), free(vd64), free(cache), free(q),
      free(out);
  return bad;
}

int main(void) {
  int bad = 0;
  bad |= run_format("q4_0", 256, 0);
  bad |= run_format("q4_0", 64, 0);
  bad |= run_format("q8_0", 128, 0);
  bad |= run_format("octave_k3v4", 128, 64);
  bad |= run_format("octave_k3v3", 192, 64);
  bad |= run_format("octave_k3v3_compact", 256, 0);
  bad |= run_format("octave_k3v4", 256, 256);
  orc_format f;
  bad |= orc_format_init(&f, "octave_k3v3_compact", 192, 0) == ORC_OK; /* must be refused */
  bad |= orc_format_init(&f, "octave_k9v9", 128, 64) == ORC_OK;
  float x[256];
  uint8_t codes[256], packed[128];
  for (int i = 0; i < 256; ++i) x[i] = rnd();
  for (int n = 16; n <= 256; n *= 2) (void)orc_block_sum(x, n);
  (void)orc_block_sum(x, 192);
  orc_fwht_f32(x, 256, 128);
  for (int bits = 3; bits <= 4; ++bits) {
    float sc;
    int32_t lut[16];
    double lv[16];
    orc_lloyd_max(bits, lv);
    (void)orc_codebook(bits, lut);
    orc_quantize_lut(x, 192, bits, codes, &sc);
    orc_pack(codes, 192, bits, packed);
    orc_unpack(packed, 192, bits, codes);
  }
  uint16_t d16;
  int8_t c8[32];
  orc_q4_0_block(x, codes, &d16);
  orc_q8_0_block(x, c8, &d16);
  int32_t words[8];
  orc_sign_bits(256, words);
  printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
  return bad;
}
