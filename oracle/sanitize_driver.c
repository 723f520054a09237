/*
 * sanitize_driver.c -- runs every oracle entry point on small seeded inputs so that a build
 * of pnmix_oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (gcc) can check it
 * for out-of-bounds accesses, leaks and undefined arithmetic.  TEST INFRASTRUCTURE ONLY: built
 * and run by tests/test_oracle_sanitize.py; it checks no values (the pins do that).
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pnmix_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* splitmix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}
/* a finite fp16 value of moderate size */
static uint16_t rnd_f16(void) {
  float f = ((float)(next_u32() % 20001) - 10000.0f) / 1000.0f;
  return orc_f2h(f);
}

static int run_cfg(orc_cfg c, int P, int sink_len, int n_pages, int res_len) {
  const int d = c.d, N = c.N, words = orc_mask_words(&c);
  const int64_t kpb = orc_k_page_bytes(&c), vpb = orc_v_page_bytes(&c);
  int rc = 0;
  uint16_t* q = malloc(sizeof(uint16_t) * (size_t)c.H_q * P * d);
  uint16_t* k = malloc(sizeof(uint16_t) * (size_t)c.H_kv * P * d);
  for (int64_t i = 0; i < (int64_t)c.H_q * P * d; ++i) q[i] = rnd_f16();
  for (int64_t i = 0; i < (int64_t)c.H_kv * P * d; ++i) k[i] = rnd_f16();
  float* qm = malloc(sizeof(float) * (size_t)c.H_q * (d / 2));
  float* km = malloc(sizeof(float) * (size_t)c.H_kv * (d / 2));
  float* sg = malloc(sizeof(float) * (size_t)c.H_kv * (d / 2));
  uint32_t* mask = malloc(sizeof(uint32_t) * (size_t)c.H_kv * words);
  rc |= orc_score_prefill(&c, P, q, k, qm, km, sg, mask);
  const int mp = n_pages > 0 ? n_pages : 1;
  uint8_t* kp = calloc((size_t)c.H_kv * mp, (size_t)kpb);
  uint8_t* vp = calloc((size_t)c.H_kv * mp, (size_t)vpb);
  uint16_t* page = malloc(sizeof(uint16_t) * (size_t)N * d);
  double* dq = malloc(sizeof(double) * (size_t)N * d);
  uint8_t* codes = malloc((size_t)N * d);
  uint16_t* S = malloc(sizeof(uint16_t) * (size_t)N * d);
  uint16_t* Z = malloc(sizeof(uint16_t) * (size_t)N * d);
  for (int h = 0; h < c.H_kv; ++h)
    for (int p = 0; p < n_pages; ++p) {
      for (int i = 0; i < N * d; ++i) page[i] = rnd_f16();
      for (int t = 0; t < N; ++t) page[t * d] = page[0]; /* a constant key channel */
      rc |= orc_quantize_k_page(&c, page, d, mask + (int64_t)h * words, kp + ((int64_t)h * mp + p) * kpb);
      rc |= orc_quantize_v_page(&c, page, d, vp + ((int64_t)h * mp + p) * vpb);
      rc |= orc_unpack_k_page(&c, kp + ((int64_t)h * mp + p) * kpb, mask + (int64_t)h * words, codes, S, Z);
      if (c.b_V != 16) rc |= orc_unpack_v_page(&c, vp + ((int64_t)h * mp + p) * vpb, codes, S, Z);
      rc |= orc_dequant_k_page(&c, kp + ((int64_t)h * mp + p) * kpb, mask + (int64_t)h * words, dq);
      rc |= orc_dequant_v_page(&c, vp + ((int64_t)h * mp + p) * vpb, dq);
    }
  uint16_t* ks = calloc((size_t)c.H_kv * (c.N_s > 0 ? c.N_s : 1) * d, sizeof(uint16_t));
  uint16_t* vs = calloc((size_t)c.H_kv * (c.N_s > 0 ? c.N_s : 1) * d, sizeof(uint16_t));
  uint16_t* kr = calloc((size_t)c.H_kv * N * d, sizeof(uint16_t));
  uint16_t* vr = calloc((size_t)c.H_kv * N * d, sizeof(uint16_t));
  for (int64_t i = 0; i < (int64_t)c.H_kv * c.N_s * d; ++i) ks[i] = vs[i] = rnd_f16();
  for (int64_t i = 0; i < (int64_t)c.H_kv * N * d; ++i) kr[i] = vr[i] = rnd_f16();
  double* out = malloc(sizeof(double) * (size_t)c.H_q * d);
  rc |= orc_decode_attn_f64(&c, sink_len, n_pages, res_len, mp, q, ks, vs, kp, vp, kr, vr, mask,
                            1.0 / sqrt((double)d), out);
  free(q); free(k); free(qm); free(km); free(sg); free(mask); free(kp); free(vp); free(page);
  free(dq); free(codes); free(S); free(Z); free(ks); free(vs); free(kr); free(vr); free(out);
  return rc;
}

int main(void) {
  int rc = 0;
  /* fp16 conversions and pair norms over every fp16 pattern */
  for (uint32_t h = 0; h < 65536; ++h) {
    volatile float f = orc_h2f((uint16_t)h);
    (void)orc_f2h(f);
    (void)orc_pair_norm((uint16_t)h, (uint16_t)(h * 2654435761u >> 16));
  }
  const orc_cfg cfgs[] = {
      /* H_q H_kv d pairing n_hi G b_H b_L b_V g_V N_s N */
      {4, 2, 32, 0, 8, 128, 3, 1, 2, 32, 32, 128},
      {8, 2, 64, 1, 12, 64, 3, 1, 2, 16, 32, 128},
      {8, 1, 128, 1, 25, 64, 3, 1, 2, 32, 32, 128},
      {4, 2, 64, 1, 10, 32, 4, 2, 4, 32, 16, 64},
      {4, 4, 32, 0, 4, 16, 4, 3, 1, 8, 0, 32},
      {2, 1, 32, 1, 0, 128, 2, 2, 16, 32, 8, 128},
      {6, 3, 64, 0, 32, 128, 1, 1, 1, 64, 32, 128},
  };
  for (size_t i = 0; i < sizeof(cfgs) / sizeof(cfgs[0]); ++i) {
    if (orc_check_cfg(&cfgs[i])) {
      fprintf(stderr, "cfg %zu rejected\n", i);
      return 2;
    }
    rc |= run_cfg(cfgs[i], 141, cfgs[i].N_s, 2, cfgs[i].N < 57 ? cfgs[i].N : 57);
    rc |= run_cfg(cfgs[i], 5, cfgs[i].N_s < 5 ? cfgs[i].N_s : 5, 0, 0 + (cfgs[i].N_s < 5));
  }
  printf("oracle sanitize driver: %s\n", rc ? "an entry point returned an error" : "ok");
  return rc ? 1 : 0;
}
