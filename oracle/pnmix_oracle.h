/*
 * pnmix_oracle.h -- plain, slow, scalar CPU oracle for the PN-Mix key-cache data path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or call this
 * file: only tests/, the smoke check in __graft_entry__.py and the cpu_baseline leg of
 * bench.py use it.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (cited by page title and section / equation):
 *   [PNMIX]  "PN-Mix: Pair-Norm Guided Mixed-Precision Key Cache Quantization for Efficient
 *            Long-Output LLM Inference" (arXiv 2610.19605): sec. 2 (GQA attention, Eq. 1;
 *            asymmetric group quantization, Eq. 2; online FP16 residual buffer), sec. 5
 *            (PN-Mix: FP16 sinks and residual buffer, Figure 1), the kernel-implementation
 *            appendix (H3/L1 bit planes, value packing, fused decode regions) and the
 *            bit-width appendix (storage accounting, T_q = 32,768).
 *   [REPRO]  "PN-Mix: Key-Cache Precision Allocation from RoPE Channel-Pair Norms"
 *            (reproduction notes): "Core equations" (Eq. 6, Eq. 2, Eq. 7, constant groups,
 *            H3/L1 packing, bit mask stored once) and "API and code mapping".
 *   [SUMMARY] the Korean summary page of the same paper: "무엇과 다른가" (procedure: GQA
 *            averaging, top-r% pairs per KV head, B x L x H_kv x (d/2)-bit mask, N_s = 32,
 *            N = 128, per-channel K groups, per-token V groups).
 *
 * Arithmetic contract (the readings the HIP path must reproduce bit for bit):
 *   - f(.) is the exact fp16 -> fp32 widening; h(.) is fp32 -> fp16 round-half-even with
 *     subnormals; every fp32 operation is one IEEE operation, never contracted into FMA.
 *   - score: per-token pair norm sqrtf(f(x)*f(x) + f(y)*f(y)); sums in 64-token chunks,
 *     ascending token order inside a chunk, chunk sums added in ascending chunk order,
 *     mean = sum / (float)P; sigma = ((sum over the group's query heads, ascending) /
 *     (float)n_g) * key_mean; top-n_hi pairs by sigma, ties to the lower pair index.
 *   - quantization: exact min and max (canonicalised: -0 -> +0); L = 2^b - 1 with b = b_H
 *     for channels of masked pairs, b_L for the others, b_V for values; s = (mx - mn) / L;
 *     inv = 1 / s (one IEEE reciprocal per group); q = clamp(rne((x - mn) * inv), 0, L);
 *     L = 1 groups store Eq. 7 metadata h((mx - mn) * 0.5f), h((3 mn + mx) * 0.25f);
 *     other groups store h(s), h(mn); constant groups store (+0, h(mn)) and codes 0.
 *   - packing: key codes split into a low plane (b_L bits of every channel) and a high plane
 *     (the b_H - b_L upper bits of the salient channels), each packing 8 consecutive tokens of
 *     a channel into as many bytes as the plane is wide; value codes packed 8 / b_V
 *     consecutive channels of one token per byte.
 *   - decode: float64 softmax attention over the dequantized cache (k = S * q + Z with the
 *     stored fp16 S and Z), token order sinks, pages, residual.
 *
 * Functions with no independent pin are marked "parity unpinned" in their comment.
 */
#ifndef PNMIX_ORACLE_H
#define PNMIX_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t H_q, H_kv, d, pairing; /* pairing 0: (2i, 2i+1); 1: (i, i + d/2) */
  int32_t n_hi_pairs;            /* floor(r * d / 2) pairs kept at b_H bits */
  int32_t G, b_H, b_L;           /* key token group; 1 <= b_L <= b_H <= 4 */
  int32_t b_V, g_V;              /* value bits (1, 2, 4, or 16 = fp16 kept) and channel group */
  int32_t N_s, N;                /* sink count and page / residual length */
} orc_cfg;

/* status: 0 ok, 1 invalid argument */
int orc_check_cfg(const orc_cfg* c);

/* fp16 <-> fp32 from the IEEE 754 binary16 / binary32 definitions */
float orc_h2f(uint16_t h);
uint16_t orc_f2h(float f);
void orc_h2f_array(const uint16_t* in, float* out, int64_t n);
void orc_f2h_array(const float* in, uint16_t* out, int64_t n);

/* one RoPE pair norm, fp32 */
float orc_pair_norm(uint16_t x, uint16_t y);
void orc_pair_norm_array(const uint16_t* x, const uint16_t* y, float* out, int64_t n);

int32_t orc_hi_pairs(double r, int32_t d);
void orc_pair_channels(const orc_cfg* c, int32_t i, int32_t* c0, int32_t* c1);
int32_t orc_mask_words(const orc_cfg* c);
int64_t orc_k_page_bytes(const orc_cfg* c);
int64_t orc_v_page_bytes(const orc_cfg* c);

/* Eq. 6 for one sequence.  q [H_q][P][d], k [H_kv][P][d] fp16 bits.
 * Outputs (any may be NULL): q_mean [H_q][d/2], k_mean [H_kv][d/2], sigma [H_kv][d/2],
 * mask [H_kv][words]. */
int orc_score_prefill(const orc_cfg* c, int32_t P, const uint16_t* q, const uint16_t* k,
                      float* q_mean, float* k_mean, float* sigma, uint32_t* mask);

/* one [N][d] page (row stride in elements) -> packed page bytes */
int orc_quantize_k_page(const orc_cfg* c, const uint16_t* src, int64_t src_row_stride,
                        const uint32_t* mask_row, uint8_t* dst);
int orc_quantize_v_page(const orc_cfg* c, const uint16_t* src, int64_t src_row_stride,
                        uint8_t* dst);

/* unpack a page: codes [N][d] (one code per byte), S and Z fp16 bits.
 * K: S, Z [N/G][d].  V: S, Z [N][d/g_V] (b_V < 16 only). */
int orc_unpack_k_page(const orc_cfg* c, const uint8_t* page, const uint32_t* mask_row,
                      uint8_t* codes, uint16_t* S, uint16_t* Z);
int orc_unpack_v_page(const orc_cfg* c, const uint8_t* page, uint8_t* codes, uint16_t* S,
                      uint16_t* Z);

/* dequantize a page to float64 [N][d]: x = S * q + Z with the stored fp16 S, Z (a b_V = 16
 * value page: the fp16 values) */
int orc_dequant_k_page(const orc_cfg* c, const uint8_t* page, const uint32_t* mask_row,
                       double* out);
int orc_dequant_v_page(const orc_cfg* c, const uint8_t* page, double* out);

/* float64 decode attention for one sequence.
 *   q      [H_q][d]
 *   k_sink, v_sink [H_kv][N_s][d]    (first sink_len rows valid)
 *   k_pages, v_pages [H_kv][max_pages][page bytes] (first n_pages valid)
 *   k_res, v_res [H_kv][N][d]        (first res_len rows valid)
 *   mask   [H_kv][words]
 *   out    [H_q][d] float64 */
int orc_decode_attn_f64(const orc_cfg* c, int32_t sink_len, int32_t n_pages, int32_t res_len,
                        int32_t max_pages, const uint16_t* q, const uint16_t* k_sink,
                        const uint16_t* v_sink, const uint8_t* k_pages, const uint8_t* v_pages,
                        const uint16_t* k_res, const uint16_t* v_res, const uint32_t* mask,
                        double sm_scale, double* out);

#ifdef __cplusplus
}
#endif
#endif
