/*
 * pnmix_oracle.c -- scalar CPU oracle for the PN-Mix key-cache data path.
 *
 * TEST INFRASTRUCTURE ONLY (see pnmix_oracle.h).  Build: gcc -O2 -ffp-contract=off
 * -fno-fast-math; x86-64 SSE arithmetic, so every float operation below is one IEEE
 * binary32 operation with round-to-nearest-even.
 *
 * Every step follows the cited passage in the pages' order; nothing is blocked, fused or
 * reordered beyond what is written in the comments.
 */
#include "pnmix_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* IEEE 754 conversions                                                                  */
/* ------------------------------------------------------------------------------------ */

/* binary16 -> binary32, exact: a binary16 value is (-1)^s * 2^(e-15) * (1 + m/1024) for
 * 0 < e < 31, (-1)^s * 2^-14 * (m/1024) for e == 0, and inf/nan for e == 31. */
float orc_h2f(uint16_t h) {
  uint32_t s = (uint32_t)(h >> 15) & 1u;
  uint32_t e = (uint32_t)(h >> 10) & 0x1fu;
  uint32_t m = (uint32_t)h & 0x3ffu;
  double v;
  if (e == 0x1f) {
    if (m == 0) return s ? -INFINITY : INFINITY;
    return s ? -NAN : NAN;
  }
  if (e == 0)
    v = ldexp((double)m, -24);
  else
    v = ldexp((double)(1024u + m), (int)e - 25);
  return (float)(s ? -v : v); /* exact: at most 11 significant bits */
}

/* binary32 -> binary16, round to nearest, ties to even, with subnormals and overflow to
 * infinity.  Written from the definition: find the binade of |f|, the spacing of binary16
 * values in it (2^(E-10), or 2^-24 below the normal range), round |f| / spacing to an
 * integer with ties to even, and encode. */
uint16_t orc_f2h(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  if (isinf(f)) return (uint16_t)(sign | 0x7c00u);
  double v = fabs((double)f);
  if (v == 0.0) return sign;
  int e2;
  frexp(v, &e2); /* v = frac * 2^e2, frac in [0.5, 1) */
  int E = e2 - 1; /* floor(log2 v) */
  if (E < -14) E = -14;
  double spacing = ldexp(1.0, E - 10);
  double n = nearbyint(v / spacing); /* exact quotient (power-of-two divisor); RNE */
  if (n >= 2048.0) { /* rounded up into the next binade */
    n = 1024.0;
    E += 1;
  }
  if (n < 1024.0) { /* subnormal (only possible when E == -14) or zero */
    return (uint16_t)(sign | (uint16_t)n);
  }
  if (E + 15 >= 31) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

void orc_h2f_array(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_h2f(in[i]);
}

void orc_f2h_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f2h(in[i]);
}

/* ------------------------------------------------------------------------------------ */
/* configuration                                                                         */
/* ------------------------------------------------------------------------------------ */

int orc_check_cfg(const orc_cfg* c) {
  if (!c) return 1;
  if (c->H_q <= 0 || c->H_kv <= 0 || c->H_q % c->H_kv) return 1;
  if (c->d <= 0 || c->d % 8 || c->d > 256) return 1;
  if (c->pairing != 0 && c->pairing != 1) return 1;
  if (c->n_hi_pairs < 0 || c->n_hi_pairs > c->d / 2) return 1;
  if (c->N <= 0 || c->N % 16) return 1;
  if (c->G <= 0 || c->N % c->G || c->G % 8) return 1;
  if (c->b_L < 1 || c->b_L > 4 || c->b_H < c->b_L || c->b_H > 4) return 1;
  if (c->b_V != 1 && c->b_V != 2 && c->b_V != 4 && c->b_V != 16) return 1;
  if (c->g_V <= 0 || c->d % c->g_V || c->g_V % 4) return 1;
  if (c->N_s < 0) return 1;
  return 0;
}

/* floor(r * d / 2) whole pairs ([REPRO] Core equations: "Select floor(r d/2) complete
 * pairs"); the 1e-9 guards r values such as 0.4 whose binary form is slightly low. */
int32_t orc_hi_pairs(double r, int32_t d) { return (int32_t)floor(r * (double)(d / 2) + 1e-9); }

/* RoPE pairing: adjacent channels (2i, 2i+1) in [PNMIX] sec. 2; split-half (i, i + d/2)
 * in the Hugging Face layout that [REPRO] distinguishes. */
void orc_pair_channels(const orc_cfg* c, int32_t i, int32_t* c0, int32_t* c1) {
  if (c->pairing == 0) {
    *c0 = 2 * i;
    *c1 = 2 * i + 1;
  } else {
    *c0 = i;
    *c1 = i + c->d / 2;
  }
}

/* d/2 mask bits per (sequence, KV head), [SUMMARY] "무엇과 다른가" */
int32_t orc_mask_words(const orc_cfg* c) { return (c->d / 2 + 31) / 32; }

static int mask_bit(const uint32_t* mask_row, int32_t pair) {
  return (int)((mask_row[pair / 32] >> (pair % 32)) & 1u);
}

/* channel c is salient when its RoPE pair is in the mask */
static int channel_salient(const orc_cfg* c, const uint32_t* mask_row, int32_t ch) {
  int32_t pair = (c->pairing == 0) ? ch / 2 : (ch % (c->d / 2));
  return mask_bit(mask_row, pair);
}

/* K page: lo plane [N/8][b_L][d] + hi plane [N/8][b_H - b_L][n_sal] + S [N/G][d] + Z [N/G][d]
 * (fp16).  With (b_H, b_L) = (3, 1) this is the LSB plane [N/8][d] and the upper-2-bit plane
 * [N/4][n_sal] of the kernel-implementation appendix. */
int64_t orc_k_page_bytes(const orc_cfg* c) {
  int64_t n_sal = 2 * (int64_t)c->n_hi_pairs;
  return (int64_t)c->N * c->d * c->b_L / 8 + (int64_t)c->N * n_sal * (c->b_H - c->b_L) / 8 +
         2 * 2 * (int64_t)(c->N / c->G) * c->d;
}

/* V page: codes [d b_V / 8][N] + S [d/g_V][N] + Z [d/g_V][N] (fp16); with b_V = 16 (values
 * kept in full precision) the page is the fp16 rows [N][d] themselves. */
int64_t orc_v_page_bytes(const orc_cfg* c) {
  if (c->b_V == 16) return 2 * (int64_t)c->N * c->d;
  return (int64_t)c->N * c->d * c->b_V / 8 + 2 * 2 * (int64_t)c->N * (c->d / c->g_V);
}

/* ------------------------------------------------------------------------------------ */
/* Eq. 6: prefill pair-norm score and the fixed pair mask                                */
/* ------------------------------------------------------------------------------------ */

/* ||(x, y)||_2 of one RoPE pair in fp32: two products, one sum, IEEE square root. */
float orc_pair_norm(uint16_t x, uint16_t y) {
  float fx = orc_h2f(x);
  float fy = orc_h2f(y);
  float a = fx * fx;
  float b = fy * fy;
  float s = a + b;
  return sqrtf(s);
}

void orc_pair_norm_array(const uint16_t* x, const uint16_t* y, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_pair_norm(x[i], y[i]);
}

/* Mean over the P prefill tokens of one head's pair norm: 64-token chunks summed in
 * ascending token order, chunk sums added in ascending chunk order, then divided by P.
 * ([REPRO] Eq. 6 E_t / E_s; [PNMIX] sec. 5: statistics of the prefill tokens.) */
static float pair_norm_mean(const orc_cfg* c, int32_t P, const uint16_t* x /*[P][d]*/,
                            int32_t pair) {
  int32_t c0, c1;
  orc_pair_channels(c, pair, &c0, &c1);
  float total = 0.0f;
  for (int32_t t0 = 0; t0 < P; t0 += 64) {
    float chunk = 0.0f;
    for (int32_t t = t0; t < t0 + 64 && t < P; ++t)
      chunk = chunk + orc_pair_norm(x[(int64_t)t * c->d + c0], x[(int64_t)t * c->d + c1]);
    total = total + chunk;
  }
  return total / (float)P;
}

/* Eq. 6 ([REPRO] Core equations; [SUMMARY] "무엇과 다른가"): for KV head h and pair i,
 * sigma = (1/|g^-1(h)|) * sum over the query heads h' sharing h of
 * E_t||q_{h',t,i}|| * E_s||k_{h,s,i}||, evaluated as ((sum of query means) / n_g) * key
 * mean.  Query head h' uses KV head floor(h' / n_g).  The top floor(r d/2) pairs of each KV
 * head (sigma descending, ties to the lower pair index) set bits of the fixed mask. */
int orc_score_prefill(const orc_cfg* c, int32_t P, const uint16_t* q, const uint16_t* k,
                      float* q_mean, float* k_mean, float* sigma, uint32_t* mask) {
  if (orc_check_cfg(c) || P <= 0 || !q || !k) return 1;
  const int32_t np = c->d / 2;
  const int32_t ng = c->H_q / c->H_kv;
  const int32_t words = orc_mask_words(c);
  float* qm = (float*)malloc(sizeof(float) * (size_t)c->H_q * np);
  float* km = (float*)malloc(sizeof(float) * (size_t)c->H_kv * np);
  float* sg = (float*)malloc(sizeof(float) * (size_t)np);
  if (!qm || !km || !sg) {
    free(qm);
    free(km);
    free(sg);
    return 1;
  }
  for (int32_t h = 0; h < c->H_q; ++h)
    for (int32_t i = 0; i < np; ++i)
      qm[h * np + i] = pair_norm_mean(c, P, q + (int64_t)h * P * c->d, i);
  for (int32_t h = 0; h < c->H_kv; ++h)
    for (int32_t i = 0; i < np; ++i)
      km[h * np + i] = pair_norm_mean(c, P, k + (int64_t)h * P * c->d, i);
  if (q_mean) memcpy(q_mean, qm, sizeof(float) * (size_t)c->H_q * np);
  if (k_mean) memcpy(k_mean, km, sizeof(float) * (size_t)c->H_kv * np);

  for (int32_t h = 0; h < c->H_kv; ++h) {
    for (int32_t i = 0; i < np; ++i) {
      float a = 0.0f;
      for (int32_t hq = h * ng; hq < h * ng + ng; ++hq) a = a + qm[hq * np + i];
      sg[i] = (a / (float)ng) * km[h * np + i];
    }
    if (sigma) memcpy(sigma + (int64_t)h * np, sg, sizeof(float) * (size_t)np);
    if (mask) {
      uint32_t* row = mask + (int64_t)h * words;
      for (int32_t w = 0; w < words; ++w) row[w] = 0u;
      for (int32_t i = 0; i < np; ++i) {
        int32_t rank = 0;
        for (int32_t j = 0; j < np; ++j)
          if (sg[j] > sg[i] || (sg[j] == sg[i] && j < i)) rank++;
        if (rank < c->n_hi_pairs) row[i / 32] |= 1u << (i % 32);
      }
    }
  }
  free(qm);
  free(km);
  free(sg);
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Eq. 2 / Eq. 7 group quantizer                                                         */
/* ------------------------------------------------------------------------------------ */

typedef struct {
  uint16_t S, Z; /* stored fp16 metadata */
} group_meta;

/* Quantize one group of n values (fp16 bits at stride) with L = 2^b - 1 levels.
 *   Eq. 2 ([PNMIX] sec. 2; [REPRO] Core equations): s = (max - min)/(2^b - 1), z = min,
 *         q = clip(round((x - z)/s), 0, 2^b - 1).  round is half-to-even; (x - z)/s is
 *         evaluated as (x - z) * (1/s) with one IEEE reciprocal per group.
 *   Eq. 7 ([REPRO]): a 1-bit group stores s = (max - min)/2, z = (3 min + max)/4, which
 *         moves its two levels to the bin midpoints; the codes are those of Eq. 2.
 *   Constant groups ([REPRO]): zero scale, the original offset, codes 0. */
static group_meta quantize_group(const uint16_t* x, int64_t stride, int32_t n, int32_t bits,
                                 uint8_t* codes, int64_t code_stride) {
  const int32_t L = (1 << bits) - 1;
  float mn = orc_h2f(x[0]);
  float mx = mn;
  for (int32_t i = 1; i < n; ++i) {
    float v = orc_h2f(x[i * stride]);
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  mn = mn + 0.0f; /* -0 -> +0 */
  mx = mx + 0.0f;
  group_meta m;
  if (mx == mn) {
    for (int32_t i = 0; i < n; ++i) codes[i * code_stride] = 0;
    m.S = 0;
    m.Z = orc_f2h(mn);
    return m;
  }
  float s = (mx - mn) / (float)L;
  float inv = 1.0f / s;
  for (int32_t i = 0; i < n; ++i) {
    float v = orc_h2f(x[i * stride]);
    float t = (v - mn) * inv;
    float r = nearbyintf(t);
    if (r < 0.0f) r = 0.0f;
    if (r > (float)L) r = (float)L;
    codes[i * code_stride] = (uint8_t)(int32_t)r;
  }
  if (L == 1) {
    float s7 = (mx - mn) * 0.5f;
    float t3 = 3.0f * mn;
    float z7 = (t3 + mx) * 0.25f;
    m.S = orc_f2h(s7);
    m.Z = orc_f2h(z7);
  } else {
    m.S = orc_f2h(s);
    m.Z = orc_f2h(mn);
  }
  return m;
}

static void put_f16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xff);
  p[1] = (uint8_t)(v >> 8);
}

static uint16_t get_f16(const uint8_t* p) { return (uint16_t)(p[0] | ((uint16_t)p[1] << 8)); }

/* Token bit plane of width w bits ([PNMIX] kernel-implementation appendix: the LSB of a key
 * channel is packed 8 consecutive tokens per byte, its upper 2 bits 4 consecutive tokens per
 * byte).  Generalised to any width w: the w-bit fields of 8 consecutive tokens 8j..8j+7 of one
 * column form an 8w-bit little-endian stream (token 8j+k at bits wk..wk+w-1), stored as w bytes
 * [j][0..w-1] of that column; plane bytes are arranged [N/8][w][ncols].  For w = 1 this is the
 * LSB byte of 8 tokens, for w = 2 two bytes of 4 tokens each. */
static void plane_put(uint8_t* plane, int32_t ncols, int32_t w, int32_t col, int32_t t,
                      uint32_t field) {
  int32_t j = t / 8, k = t % 8;
  for (int32_t bit = 0; bit < w; ++bit) {
    int32_t pos = w * k + bit; /* position in the 8w-bit stream */
    if ((field >> bit) & 1u)
      plane[((int64_t)j * w + pos / 8) * ncols + col] |= (uint8_t)(1u << (pos % 8));
  }
}

static uint32_t plane_get(const uint8_t* plane, int32_t ncols, int32_t w, int32_t col,
                          int32_t t) {
  int32_t j = t / 8, k = t % 8;
  uint32_t field = 0;
  for (int32_t bit = 0; bit < w; ++bit) {
    int32_t pos = w * k + bit;
    field |= (uint32_t)((plane[((int64_t)j * w + pos / 8) * ncols + col] >> (pos % 8)) & 1u)
             << bit;
  }
  return field;
}

/* K page ([PNMIX] kernel-implementation appendix; [REPRO] H3/L1 packing; [SUMMARY]):
 * keys are quantized per channel over token groups of G; channels of salient pairs use
 * b_H bits, the rest b_L bits (Eq. 7 for any 1-bit group).  The low b_L bits of every
 * channel's code go to the lo plane (width b_L, all d channels); the upper b_H - b_L bits of
 * the salient channels go to the hi plane (width b_H - b_L, n_sal columns, salient channels in
 * ascending channel order = rank r):
 *     lo [N/8][b_L][d]            field of (t, c) = q(t, c) & (2^b_L - 1)
 *     hi [N/8][b_H - b_L][n_sal]  field of (t, r) = q(t, sal(r)) >> b_L
 * then S[g][c] and Z[g][c] as little-endian fp16 ([N/G][d] each).  With (b_H, b_L) = (3, 1):
 * lo byte [j][c] bit k = q(8j + k, c) & 1 and hi byte [j][r] bits 2k..2k+1 = q(4j + k, sal(r))
 * >> 1, the appendix's two planes. */
int orc_quantize_k_page(const orc_cfg* c, const uint16_t* src, int64_t src_row_stride,
                        const uint32_t* mask_row, uint8_t* dst) {
  if (orc_check_cfg(c) || !src || !mask_row || !dst) return 1;
  const int32_t N = c->N, d = c->d, G = c->G, ngr = N / G;
  const int32_t n_sal = 2 * c->n_hi_pairs;
  const int32_t wL = c->b_L, wH = c->b_H - c->b_L;
  int32_t cnt = 0;
  for (int32_t ch = 0; ch < d; ++ch) cnt += channel_salient(c, mask_row, ch);
  if (cnt != n_sal) return 1; /* mask popcount must equal n_hi_pairs */
  uint8_t* codes = (uint8_t*)malloc((size_t)N * d);
  if (!codes) return 1;
  uint8_t* lo = dst;
  uint8_t* hi = dst + (int64_t)N * d * wL / 8;
  uint8_t* Sp = hi + (int64_t)N * n_sal * wH / 8;
  uint8_t* Zp = Sp + 2 * (int64_t)ngr * d;
  for (int32_t g = 0; g < ngr; ++g) {
    for (int32_t ch = 0; ch < d; ++ch) {
      int bits = channel_salient(c, mask_row, ch) ? c->b_H : c->b_L;
      group_meta m = quantize_group(src + (int64_t)g * G * src_row_stride + ch, src_row_stride,
                                    G, bits, codes + (int64_t)g * G * d + ch, d);
      put_f16(Sp + 2 * ((int64_t)g * d + ch), m.S);
      put_f16(Zp + 2 * ((int64_t)g * d + ch), m.Z);
    }
  }
  memset(lo, 0, (size_t)N * d * wL / 8);
  memset(hi, 0, (size_t)N * n_sal * wH / 8);
  for (int32_t t = 0; t < N; ++t)
    for (int32_t ch = 0; ch < d; ++ch)
      plane_put(lo, d, wL, ch, t, codes[t * d + ch] & ((1u << wL) - 1u));
  if (wH > 0) {
    int32_t r = 0;
    for (int32_t ch = 0; ch < d; ++ch) {
      if (!channel_salient(c, mask_row, ch)) continue;
      for (int32_t t = 0; t < N; ++t) plane_put(hi, n_sal, wH, r, t, (uint32_t)codes[t * d + ch] >> wL);
      r++;
    }
  }
  free(codes);
  return 0;
}

/* V page ([PNMIX] sec. 2 and kernel-implementation appendix; [SUMMARY]): values are
 * quantized per token over channel groups of g_V at b_V bits (Eq. 2, Eq. 7 for b_V = 1, the
 * constant rule).  Consecutive channels of one token share a byte, as the appendix packs
 * 4 consecutive channel values of a token into one byte at b_V = 2: byte [m][t] holds the
 * channels e m .. e m + e - 1 of token t, e = 8 / b_V, channel e m + u in bits
 * b_V u .. b_V u + b_V - 1.  Bytes are arranged [d b_V / 8][N] (the N tokens of one byte
 * column contiguous), then S[g][t], Z[g][t] as little-endian fp16 ([d/g_V][N] each,
 * group-major).  With b_V = 16 the values stay fp16 and the page is the rows [N][d]. */
int orc_quantize_v_page(const orc_cfg* c, const uint16_t* src, int64_t src_row_stride,
                        uint8_t* dst) {
  if (orc_check_cfg(c) || !src || !dst) return 1;
  const int32_t N = c->N, d = c->d, ng = d / c->g_V, bV = c->b_V;
  if (bV == 16) {
    for (int32_t t = 0; t < N; ++t)
      for (int32_t ch = 0; ch < d; ++ch)
        put_f16(dst + 2 * ((int64_t)t * d + ch), src[(int64_t)t * src_row_stride + ch]);
    return 0;
  }
  const int32_t e = 8 / bV; /* channels per byte */
  uint8_t* codes = (uint8_t*)malloc((size_t)N * d);
  if (!codes) return 1;
  uint8_t* cb = dst;
  uint8_t* Sp = dst + (int64_t)N * d * bV / 8;
  uint8_t* Zp = Sp + 2 * (int64_t)N * ng;
  for (int32_t t = 0; t < N; ++t) {
    for (int32_t g = 0; g < ng; ++g) {
      group_meta m = quantize_group(src + (int64_t)t * src_row_stride + g * c->g_V, 1, c->g_V,
                                    bV, codes + (int64_t)t * d + g * c->g_V, 1);
      put_f16(Sp + 2 * ((int64_t)g * N + t), m.S);
      put_f16(Zp + 2 * ((int64_t)g * N + t), m.Z);
    }
  }
  memset(cb, 0, (size_t)N * d * bV / 8);
  for (int32_t t = 0; t < N; ++t)
    for (int32_t ch = 0; ch < d; ++ch)
      cb[(int64_t)(ch / e) * N + t] |= (uint8_t)(codes[t * d + ch] << (bV * (ch % e)));
  free(codes);
  return 0;
}

/* ------------------------------------------------------------------------------------ */
/* unpacking and dequantization (inverse of the layouts above)                           */
/* ------------------------------------------------------------------------------------ */

int orc_unpack_k_page(const orc_cfg* c, const uint8_t* page, const uint32_t* mask_row,
                      uint8_t* codes, uint16_t* S, uint16_t* Z) {
  if (orc_check_cfg(c) || !page || !mask_row) return 1;
  const int32_t N = c->N, d = c->d, ngr = N / c->G;
  const int32_t n_sal = 2 * c->n_hi_pairs;
  const int32_t wL = c->b_L, wH = c->b_H - c->b_L;
  const uint8_t* lo = page;
  const uint8_t* hi = page + (int64_t)N * d * wL / 8;
  const uint8_t* Sp = hi + (int64_t)N * n_sal * wH / 8;
  const uint8_t* Zp = Sp + 2 * (int64_t)ngr * d;
  if (codes) {
    for (int32_t t = 0; t < N; ++t)
      for (int32_t ch = 0; ch < d; ++ch) codes[t * d + ch] = (uint8_t)plane_get(lo, d, wL, ch, t);
    if (wH > 0) {
      int32_t r = 0;
      for (int32_t ch = 0; ch < d; ++ch) {
        if (!channel_salient(c, mask_row, ch)) continue;
        for (int32_t t = 0; t < N; ++t)
          codes[t * d + ch] |= (uint8_t)(plane_get(hi, n_sal, wH, r, t) << wL);
        r++;
      }
    }
  }
  for (int32_t i = 0; i < ngr * d; ++i) {
    if (S) S[i] = get_f16(Sp + 2 * i);
    if (Z) Z[i] = get_f16(Zp + 2 * i);
  }
  return 0;
}

/* b_V < 16 only (a b_V = 16 page holds no codes) */
int orc_unpack_v_page(const orc_cfg* c, const uint8_t* page, uint8_t* codes, uint16_t* S,
                      uint16_t* Z) {
  if (orc_check_cfg(c) || !page || c->b_V == 16) return 1;
  const int32_t N = c->N, d = c->d, ng = d / c->g_V, bV = c->b_V, e = 8 / bV;
  const uint8_t* cb = page;
  const uint8_t* Sp = page + (int64_t)N * d * bV / 8;
  const uint8_t* Zp = Sp + 2 * (int64_t)N * ng;
  if (codes)
    for (int32_t t = 0; t < N; ++t)
      for (int32_t ch = 0; ch < d; ++ch)
        codes[t * d + ch] =
            (uint8_t)((cb[(int64_t)(ch / e) * N + t] >> (bV * (ch % e))) & ((1u << bV) - 1u));
  /* S, Z are returned per token, [N][d/g_V], from the group-major storage */
  for (int32_t t = 0; t < N; ++t)
    for (int32_t g = 0; g < ng; ++g) {
      if (S) S[t * ng + g] = get_f16(Sp + 2 * ((int64_t)g * N + t));
      if (Z) Z[t * ng + g] = get_f16(Zp + 2 * ((int64_t)g * N + t));
    }
  return 0;
}

/* reconstruction x = s q + z of Eq. 2 with the stored fp16 metadata, in float64 */
int orc_dequant_k_page(const orc_cfg* c, const uint8_t* page, const uint32_t* mask_row,
                       double* out) {
  if (orc_check_cfg(c) || !page || !mask_row || !out) return 1;
  const int32_t N = c->N, d = c->d, G = c->G, ngr = N / G;
  uint8_t* codes = (uint8_t*)malloc((size_t)N * d);
  uint16_t* S = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)ngr * d);
  uint16_t* Z = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)ngr * d);
  int rc = (!codes || !S || !Z) ? 1 : orc_unpack_k_page(c, page, mask_row, codes, S, Z);
  if (rc == 0)
    for (int32_t t = 0; t < N; ++t)
      for (int32_t ch = 0; ch < d; ++ch) {
        int32_t g = t / G;
        out[(int64_t)t * d + ch] = (double)orc_h2f(S[g * d + ch]) * (double)codes[t * d + ch] +
                                   (double)orc_h2f(Z[g * d + ch]);
      }
  free(codes);
  free(S);
  free(Z);
  return rc;
}

int orc_dequant_v_page(const orc_cfg* c, const uint8_t* page, double* out) {
  if (orc_check_cfg(c) || !page || !out) return 1;
  const int32_t N = c->N, d = c->d, ng = d / c->g_V;
  if (c->b_V == 16) {
    for (int64_t i = 0; i < (int64_t)N * d; ++i) out[i] = (double)orc_h2f(get_f16(page + 2 * i));
    return 0;
  }
  uint8_t* codes = (uint8_t*)malloc((size_t)N * d);
  uint16_t* S = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N * ng);
  uint16_t* Z = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)N * ng);
  int rc = (!codes || !S || !Z) ? 1 : orc_unpack_v_page(c, page, codes, S, Z);
  if (rc == 0)
    for (int32_t t = 0; t < N; ++t)
      for (int32_t ch = 0; ch < d; ++ch) {
        int32_t g = ch / c->g_V;
        out[(int64_t)t * d + ch] = (double)orc_h2f(S[t * ng + g]) * (double)codes[t * d + ch] +
                                   (double)orc_h2f(Z[t * ng + g]);
      }
  free(codes);
  free(S);
  free(Z);
  return rc;
}

/* ------------------------------------------------------------------------------------ */
/* decode attention, float64                                                             */
/* ------------------------------------------------------------------------------------ */

/* Eq. 1 ([PNMIX] sec. 2) at one decode position, over the cache of sec. 5 and the
 * kernel-implementation appendix: FP16 sinks, then the dequantized pages, then the FP16
 * residual buffer.  Each KV head's cache is dequantized densely to float64 first, then
 * logits = (q . k) * sm_scale, p = softmax(logits), out = sum p v.  Query head h' reads
 * KV head floor(h' / n_g). */
int orc_decode_attn_f64(const orc_cfg* c, int32_t sink_len, int32_t n_pages, int32_t res_len,
                        int32_t max_pages, const uint16_t* q, const uint16_t* k_sink,
                        const uint16_t* v_sink, const uint8_t* k_pages, const uint8_t* v_pages,
                        const uint16_t* k_res, const uint16_t* v_res, const uint32_t* mask,
                        double sm_scale, double* out) {
  if (orc_check_cfg(c) || !q || !out) return 1;
  if (sink_len < 0 || sink_len > c->N_s || res_len < 0 || res_len > c->N || n_pages < 0 ||
      n_pages > max_pages)
    return 1;
  const int32_t d = c->d, N = c->N, ng = c->H_q / c->H_kv;
  const int64_t T = (int64_t)sink_len + (int64_t)n_pages * N + res_len;
  const int64_t kpb = orc_k_page_bytes(c), vpb = orc_v_page_bytes(c);
  const int32_t words = orc_mask_words(c);
  if (T == 0) return 1;
  double* K = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* V = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* lg = (double*)malloc(sizeof(double) * (size_t)T);
  if (!K || !V || !lg) {
    free(K);
    free(V);
    free(lg);
    return 1;
  }
  int rc = 0;
  for (int32_t h = 0; h < c->H_kv && rc == 0; ++h) {
    int64_t t = 0;
    for (int32_t i = 0; i < sink_len; ++i, ++t)
      for (int32_t ch = 0; ch < d; ++ch) {
        K[t * d + ch] = (double)orc_h2f(k_sink[((int64_t)h * c->N_s + i) * d + ch]);
        V[t * d + ch] = (double)orc_h2f(v_sink[((int64_t)h * c->N_s + i) * d + ch]);
      }
    for (int32_t p = 0; p < n_pages && rc == 0; ++p) {
      rc |= orc_dequant_k_page(c, k_pages + ((int64_t)h * max_pages + p) * kpb,
                               mask + (int64_t)h * words, K + t * d);
      rc |= orc_dequant_v_page(c, v_pages + ((int64_t)h * max_pages + p) * vpb, V + t * d);
      t += N;
    }
    for (int32_t i = 0; i < res_len; ++i, ++t)
      for (int32_t ch = 0; ch < d; ++ch) {
        K[t * d + ch] = (double)orc_h2f(k_res[((int64_t)h * N + i) * d + ch]);
        V[t * d + ch] = (double)orc_h2f(v_res[((int64_t)h * N + i) * d + ch]);
      }
    for (int32_t hq = h * ng; hq < h * ng + ng; ++hq) {
      double m = -INFINITY;
      for (int64_t s = 0; s < T; ++s) {
        double acc = 0.0;
        for (int32_t ch = 0; ch < d; ++ch)
          acc += (double)orc_h2f(q[(int64_t)hq * d + ch]) * K[s * d + ch];
        lg[s] = acc * sm_scale;
        if (lg[s] > m) m = lg[s];
      }
      double l = 0.0;
      for (int64_t s = 0; s < T; ++s) {
        lg[s] = exp(lg[s] - m);
        l += lg[s];
      }
      for (int32_t ch = 0; ch < d; ++ch) {
        double o = 0.0;
        for (int64_t s = 0; s < T; ++s) o += lg[s] * V[s * d + ch];
        out[(int64_t)hq * d + ch] = o / l;
      }
    }
  }
  free(K);
  free(V);
  free(lg);
  return rc;
}
