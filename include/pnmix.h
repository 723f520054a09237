/*
 * pnmix.h -- C ABI of the MI355X (gfx950) PN-Mix key-cache library, libpnmix.so.
 *
 * PN-Mix keeps the key cache of a RoPE decoder in mixed precision: RoPE channel pairs with a
 * large query-key pair-norm product get b_H = 3 bits, the rest b_L = 1 bit with a midpoint
 * correction, selected once at prefill; values are quantized per token at b_V = 2 bits; the
 * first N_s tokens (sinks) and an N-token residual buffer stay in fp16.  The other bit widths of
 * the paper's sweep (Table 14 / Figure 3: b_H, b_L in {1..4}, b_V = 16 values kept in fp16, and
 * b_V in {1, 4}) are supported too, through plainer kernels.  Sources:
 *   [PNMIX]   "PN-Mix: Pair-Norm Guided Mixed-Precision Key Cache Quantization for Efficient
 *             Long-Output LLM Inference" (arXiv 2610.19605), sec. 2 (Eq. 1 GQA attention,
 *             Eq. 2 asymmetric group quantization, online residual buffer), sec. 5 (method,
 *             Figure 1), kernel-implementation appendix (bit planes, value packing, fused
 *             dequantizing decode over sink / quantized / residual regions).
 *   [REPRO]   "PN-Mix: Key-Cache Precision Allocation from RoPE Channel-Pair Norms",
 *             Core equations (Eq. 6, Eq. 2, Eq. 7, constant groups, H3/L1 packing) and
 *             "API and code mapping" (post-RoPE [batch, heads, tokens, head_dim] inputs, query
 *             heads ordered by GQA group, one cache per layer).
 *   [SUMMARY] Korean summary page of the same paper, "무엇과 다른가" (B x L x H_kv x d/2-bit
 *             mask, N_s = 32, N = 128).
 *   [FLASH]   TriAxialKV fact sheet: flash-decoding splits merged by online log-sum-exp.
 *
 * Conventions (all entry points):
 *   - Every array argument is DEVICE memory unless stated; the caller owns all memory; the
 *     library allocates nothing and keeps no state between calls.
 *   - fp16 arrays are passed as uint16_t bit patterns (IEEE binary16).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work and return
 *     without synchronising; outputs are valid when the stream reaches that point and inputs
 *     must stay unchanged until then.  Calls do not block and are thread-safe.
 *   - Arguments are validated on the host before any launch.  A failure returns a non-zero
 *     status, launches nothing and sets a thread-local message (pnmix_last_error).  HIP launch
 *     errors return PNMIX_E_HIP.  There is no CPU fallback.
 *   - Layers are folded into the batch: a "sequence" is one (layer, batch row) cache.
 *   - Device data outside the contract (NaN/Inf inputs, lengths beyond capacity, a mask whose
 *     popcount differs from n_hi_pairs) gives undefined results but never out-of-range
 *     accesses: lengths are clamped to the capacities passed in.
 */
#ifndef PNMIX_H
#define PNMIX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PNMIX_OK = 0,
  PNMIX_E_INVALID = 1,     /* null pointer, bad size, inconsistent configuration */
  PNMIX_E_UNSUPPORTED = 2, /* valid PN-Mix setting this library does not implement */
  PNMIX_E_WORKSPACE = 3,   /* workspace smaller than the *_workspace_bytes query */
  PNMIX_E_HIP = 4          /* HIP runtime or launch error (including: no device) */
} pnmix_status;

typedef enum {
  PNMIX_PAIRS_ADJACENT = 0,  /* pair i = channels (2i, 2i+1)      [PNMIX] sec. 2 */
  PNMIX_PAIRS_SPLIT_HALF = 1 /* pair i = channels (i, i + d/2)    [REPRO] */
} pnmix_pairing;

/* Problem statement of one attention layer ([PNMIX] sec. 2 and 5; [REPRO]).
 * Supported: H_q % H_kv == 0 with n_g = H_q / H_kv <= 16; d in {32, 64, 128};
 * 0 <= n_hi_pairs <= d/2; N == 128; G in {32, 64, 128}; 1 <= b_L <= b_H <= 4;
 * b_V in {1, 2, 4, 16}; g_V in {16, 32, 64, 128} dividing d with d / g_V <= 4 value groups per
 * token; 0 <= N_s <= 128.  (b_H, b_L, b_V) = (3, 1, 2) with g_V >= 32 runs on the matrix-core
 * decode kernel; every other setting decodes on the generic kernel (same results contract). */
typedef struct {
  int32_t H_q, H_kv, d, pairing;
  int32_t n_hi_pairs; /* floor(r * d / 2): pnmix_hi_pairs(r, d) */
  int32_t G, b_H, b_L;
  int32_t b_V, g_V;
  int32_t N_s, N;
} pnmix_cfg;

/* One page job: N consecutive fp16 token rows of one (sequence, KV head) -> one packed page.
 * src row t (t < N) starts at src + t * src_row_stride (elements; each row d contiguous
 * fp16); dst receives pnmix_k_page_bytes / pnmix_v_page_bytes bytes (16-byte aligned);
 * mask_row selects the mask row [mask_words] of the job's (sequence, KV head) (K only). */
typedef struct {
  const uint16_t* src;
  int64_t src_row_stride;
  uint8_t* dst;
  int64_t mask_row;
} pnmix_page;

/* Cache length of one sequence: sink_len <= N_s fp16 sinks, n_pages <= max_pages packed
 * pages of N tokens, res_len <= N fp16 residual rows; token order sinks, pages, residual. */
typedef struct {
  int32_t sink_len, n_pages, res_len, _pad;
} pnmix_seq_len;

/* ---- host-only queries ------------------------------------------------------------------- */

/* PNMIX_OK when the configuration is supported (else a status and a message). */
pnmix_status pnmix_check_cfg(const pnmix_cfg* cfg);
/* floor(r * d/2) complete pairs ([REPRO] Core equations), with a 1e-9 guard against r values
 * whose binary form lies just below the decimal one (e.g. 0.4). */
int32_t pnmix_hi_pairs(double r, int32_t d);
/* uint32 words per (sequence, KV head) of the pair mask: ceil((d/2) / 32); bit i = pair i. */
size_t pnmix_mask_words(const pnmix_cfg* cfg);
/* K page: N*d*b_L/8 (low plane) + N*2*n_hi_pairs*(b_H-b_L)/8 (high plane) + 4*(N/G)*d (fp16
 * S, Z); with (3, 1) the LSB plane N*d/8 and the upper-2-bit plane N*2*n_hi_pairs/4. */
size_t pnmix_k_page_bytes(const pnmix_cfg* cfg);
/* V page: N*d*b_V/8 (codes) + 4*N*(d/g_V) (fp16 S, Z); b_V = 16: the fp16 rows, 2*N*d. */
size_t pnmix_v_page_bytes(const pnmix_cfg* cfg);
/* Device workspace of pnmix_score_prefill (bytes, 256-aligned size). */
size_t pnmix_score_workspace_bytes(const pnmix_cfg* cfg, int32_t B, int32_t P);
/* Number of split-K partitions pnmix_decode_attn uses for this batch and capacity. */
int32_t pnmix_decode_splits(const pnmix_cfg* cfg, int32_t B, int32_t max_pages);
/* The split plan of pnmix_decode_attn for this batch and capacity (diagnostics; it depends on
 * the device's compute units and occupancy): out[0] partials per (sequence, KV head) (as
 * pnmix_decode_splits), out[1] waves over the packed pages, out[2] waves over the fp16 sink
 * and residual rows (0: their 32-token pieces are spread over the page waves), out[3] waves per
 * workgroup.  out: 4 int32 in host memory, written only on success.  PNMIX_E_INVALID for an
 * invalid configuration, B <= 0, max_pages < 0 or a NULL out. */
pnmix_status pnmix_decode_plan(const pnmix_cfg* cfg, int32_t B, int32_t max_pages, int32_t* out);
/* Device workspace of pnmix_decode_attn (bytes). */
size_t pnmix_decode_workspace_bytes(const pnmix_cfg* cfg, int32_t B, int32_t max_pages);
/* Message of the last failed call on this thread ("" if none). */
const char* pnmix_last_error(void);

/* ---- the path ---------------------------------------------------------------------------- */

/* Prefill saliency, Eq. 6 ([REPRO] Core equations; [SUMMARY]; [PNMIX] sec. 5).
 *   q    [B][H_q][P][d]  fp16, post-RoPE, query heads ordered by GQA group
 *   k    [B][H_kv][P][d] fp16, post-RoPE
 *   sigma [B][H_kv][d/2] fp32 out, or NULL
 *   mask  [B][H_kv][mask_words] uint32 out: bit i set for the floor(r d/2) pairs of largest
 *         sigma (ties to the lower pair index); stored once and reused for every page.
 * sigma_{h,i} = ((sum over the n_g query heads h' of KV head h of mean_t ||q_{h',t,i}||) / n_g)
 *               * mean_s ||k_{h,s,i}||, over all P prefill tokens (sinks included); pair norms
 * in fp32 with IEEE sqrt; each mean is the sum of 64-token chunk sums (ascending tokens, then
 * ascending chunks) divided by P.  Bit-exact with the reference oracle.
 * ws: pnmix_score_workspace_bytes(cfg, B, P) bytes of device scratch. */
pnmix_status pnmix_score_prefill(const pnmix_cfg* cfg, int32_t B, int32_t P, const uint16_t* q,
                                 const uint16_t* k, float* sigma, uint32_t* mask, void* ws,
                                 size_t ws_bytes, void* stream);

/* Prefill in one pass over the keys: pnmix_score_prefill (sigma, mask) and the quantization of
 * the prompt's full pages (tokens N_s + N p .. N_s + N p + N - 1 of every (sequence, KV head),
 * p < n_full = (P - N_s) / N) into page slots 0..n_full-1, with the mask just computed ([PNMIX]
 * sec. 5: the salient pairs are chosen once at prefill and every page uses them).  Same outputs
 * bit for bit as pnmix_score_prefill followed by pnmix_quantize_kv_pages on those pages, but the
 * keys are read once: the page workgroups also form the score's key chunk sums and keep both
 * encodings a channel can take until the mask is known.  Sinks and residual rows are the
 * caller's (the rows are copied as they are).  (b_H, b_L, b_V) = (3, 1, 2) only.
 *   q [B][H_q][P][d], k, v [B][H_kv][P][d] fp16; sigma [B][H_kv][d/2] f32 or NULL;
 *   mask [B][H_kv][mask_words] out; k_pages, v_pages [B][max_pages][H_kv][page bytes] out
 *   (slots 0..n_full-1 written; may be NULL when n_full = 0);
 *   ws: pnmix_prefill_fused_workspace_bytes(cfg, B, P) bytes (score chunk sums and the
 *   candidate encodings, about 12 KB per page). */
size_t pnmix_prefill_fused_workspace_bytes(const pnmix_cfg* cfg, int32_t B, int32_t P);
pnmix_status pnmix_prefill_fused(const pnmix_cfg* cfg, int32_t B, int32_t P, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, float* sigma,
                                 uint32_t* mask, uint8_t* k_pages, uint8_t* v_pages,
                                 int32_t max_pages, void* ws, size_t ws_bytes, void* stream);

/* Key page quantization and H3/L1 packing ([PNMIX] sec. 2 Eq. 2 and kernel-implementation
 * appendix; [REPRO] Eq. 7, constant groups, H3/L1 packing).
 *   pages [n_pages] DEVICE array of jobs; mask [rows][mask_words] (row = job.mask_row).
 * Per channel c and token group g of G tokens: exact min mn and max mx (-0 -> +0);
 * L = 2^b_H - 1 if c belongs to a masked pair else 2^b_L - 1; if mx == mn: codes 0, S = +0,
 * Z = mn; else s = (mx-mn)/L, q = clamp(rne((x-mn) * (1/s)), 0, L), stored S = h(s), Z = h(mn)
 * for L > 1 and (Eq. 7) S = h((mx-mn)*0.5), Z = h((3*mn + mx)*0.25) for L = 1 (fp32, no
 * contraction, h = fp32->fp16 round-half-even).  Page layout (bytes, LSB-first bits), for
 * (b_H, b_L) = (3, 1):
 *   lo [N/8][d]      byte [j][c] bit k = q(8j+k, c) & 1
 *   hi [N/4][n_sal]  byte [j][r] bits 2k..2k+1 = q(4j+k, sal(r)) >> 1, n_sal = 2*n_hi_pairs,
 *                    salient channels in ascending channel order
 *   S  [N/G][d] fp16, then Z [N/G][d] fp16.
 * Other widths: lo [N/8][b_L][d] holds q & (2^b_L - 1) of every channel, hi
 * [N/8][b_H-b_L][n_sal] holds q >> b_L of the salient channels; in a plane of width w the w-bit
 * fields of tokens 8j..8j+7 of one column form an 8w-bit little-endian stream (token 8j+k at
 * bits wk..wk+w-1) stored as its w bytes [j][0..w-1].
 * Bit-exact with the reference oracle. */
pnmix_status pnmix_quantize_k_page(const pnmix_cfg* cfg, int32_t n_pages,
                                   const pnmix_page* pages, const uint32_t* mask, void* stream);

/* Value page quantization and packing ([PNMIX] sec. 2 and kernel-implementation appendix:
 * every 4 consecutive channel values of a token in one byte; [SUMMARY]): per token and channel
 * group of g_V channels, Eq. 2 at b_V bits with the constant rule (Eq. 7 metadata for b_V = 1);
 * stored S = h(s), Z = h(mn).  Layout for b_V = 2:
 *   codes [d/4][N]  byte [m][t] = channels 4m..4m+3 of token t, channel 4m+u in bits 2u..2u+1
 *                   (the N tokens of one byte column contiguous)
 *   S [d/g_V][N] fp16, then Z [d/g_V][N] fp16 (group-major: one group's N tokens contiguous).
 * b_V in {1, 4}: codes [d*b_V/8][N], byte [m][t] = the 8/b_V channels (8/b_V) m + u of token t
 * in bits b_V u ..; b_V = 16: the page is the fp16 rows [N][d].
 * Bit-exact with the reference oracle. */
pnmix_status pnmix_quantize_v_page(const pnmix_cfg* cfg, int32_t n_pages,
                                   const pnmix_page* pages, void* stream);

/* Key and value pages in one call: pnmix_quantize_k_page on k_pages and pnmix_quantize_v_page
 * on v_pages (n_pages jobs each, device arrays; mask as for the key jobs), with the same bytes
 * out, in one launch whose workgroups alternate between key and value pages (the residual
 * buffer's flush, [PNMIX] sec. 2, quantizes both at once).  Settings other than
 * (b_H, b_L, b_V) = (3, 1, 2) run as two launches. */
pnmix_status pnmix_quantize_kv_pages(const pnmix_cfg* cfg, int32_t n_pages,
                                     const pnmix_page* k_pages, const pnmix_page* v_pages,
                                     const uint32_t* mask, void* stream);

/* Decode-step GQA attention straight over the packed cache ([PNMIX] Eq. 1, kernel-implementation
 * appendix: sink region, quantized region, residual region, dequantization in registers;
 * [FLASH] split-K partials merged by online log-sum-exp).
 *   q       [B][H_q][d] fp16 (one decode query per head)
 *   k_sink, v_sink   [B][H_kv][N_s][d] fp16
 *   k_pages [B][max_pages][H_kv][pnmix_k_page_bytes], v_pages [...][pnmix_v_page_bytes]:
 *           page p of every KV head of sequence b side by side (the pool layout of
 *           pnmix_decode_attn_paged below with block b * max_pages + p);
 *           max_pages * H_kv * page bytes must stay below 2 GiB (one buffer resource spans a
 *           sequence's pages; else PNMIX_E_UNSUPPORTED)
 *   k_res, v_res     [B][H_kv][N][d] fp16
 *   lens    [B] pnmix_seq_len; mask [B][H_kv][mask_words] (the rows the pages were packed with)
 *   out     [B][H_q][d] fp32: softmax(q k^T * sm_scale) v over sinks, pages (k = S q + Z with the
 *           stored fp16 S, Z), residual; query head h' reads KV head floor(h'/n_g).
 *   ws      pnmix_decode_workspace_bytes(cfg, B, max_pages) bytes of device scratch (split-K
 *           partials); calls that share a workspace must not overlap.
 * A sequence with no tokens gets out = 0.  Accuracy: max |out - float64 reference| <= 2e-3 on
 * the supported workloads (fp32 softmax; exact integer products of codes). */
pnmix_status pnmix_decode_attn(const pnmix_cfg* cfg, int32_t B, int32_t max_pages,
                               const uint16_t* q, const uint16_t* k_sink, const uint16_t* v_sink,
                               const uint8_t* k_pages, const uint8_t* v_pages,
                               const uint16_t* k_res, const uint16_t* v_res,
                               const pnmix_seq_len* lens, const uint32_t* mask, float sm_scale,
                               float* out, void* ws, size_t ws_bytes, void* stream);

/* One decode step in one call: pnmix_append_kv then pnmix_decode_attn ([PNMIX] sec. 2: the
 * new key and value enter the FP16 residual buffer, or the sinks while those fill, and the step
 * attends over the cache that includes them), with the same outputs bit for bit and one launch
 * fewer.  The new rows join the attention straight from k_new / v_new; once every split has
 * read the cache they are written into k_sink / v_sink or k_res / v_res at the row
 * pnmix_append_kv would use, and the lengths after the append go to lens_out.
 *   k_new, v_new [B][H_kv][d] fp16
 *   lens       [B] lengths before the step (read only)
 *   lens_out   [B] lengths after the step (written); must not overlap lens
 *   the other arguments as in pnmix_decode_attn (k_sink ... v_res are written).
 * A sequence whose residual buffer already holds N rows takes no new row (lens_out = lens for
 * it), as with pnmix_append_kv. */
pnmix_status pnmix_append_decode_attn(const pnmix_cfg* cfg, int32_t B, int32_t max_pages,
                                      const uint16_t* q, const uint16_t* k_new,
                                      const uint16_t* v_new, uint16_t* k_sink, uint16_t* v_sink,
                                      const uint8_t* k_pages, const uint8_t* v_pages,
                                      uint16_t* k_res, uint16_t* v_res,
                                      const pnmix_seq_len* lens, pnmix_seq_len* lens_out,
                                      const uint32_t* mask, float sm_scale, float* out, void* ws,
                                      size_t ws_bytes, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): pnmix_decode_attn with the same arguments except the
 * workspace, whose split-K partials go to a device array the library owns instead, one per GPU
 * (pnmix_noalloc_scratch_bytes() bytes, 32 MiB, held by each GPU the library runs on until the
 * process ends).  The call allocates nothing (no hipMalloc, no allocating library routine);
 * its first call on a device looks the array's address up once (hipGetSymbolAddress).
 * Results are those of pnmix_decode_attn, bit for bit.  A batch whose partials exceed the
 * array (pnmix_decode_workspace_bytes(cfg, B, max_pages) > pnmix_noalloc_scratch_bytes())
 * returns PNMIX_E_WORKSPACE before any launch.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams, or threads) race and must be serialised by
 * the caller.  Nothing in the array needs to start at zero (every partial is written before it
 * is read). */
size_t pnmix_noalloc_scratch_bytes(void);
pnmix_status pnmix_decode_attn_noalloc(const pnmix_cfg* cfg, int32_t B, int32_t max_pages,
                                       const uint16_t* q, const uint16_t* k_sink,
                                       const uint16_t* v_sink, const uint8_t* k_pages,
                                       const uint8_t* v_pages, const uint16_t* k_res,
                                       const uint16_t* v_res, const pnmix_seq_len* lens,
                                       const uint32_t* mask, float sm_scale, float* out,
                                       void* stream);

/* Decode attention over pages held in a shared pool through a block table ([BLOG] "How it
 * composes with paging, GQA and offload": a page of the quantized cache is a fixed-size block
 * carrying its own scales, so quantized pages slot into paged attention's block pool).  Same
 * operation, arithmetic and results as pnmix_decode_attn above, bit for bit: only the address
 * of page p of sequence b changes.
 *   k_pool   [n_blocks][H_kv][pnmix_k_page_bytes] u8: block i holds one page of every KV head
 *   v_pool   [n_blocks][H_kv][pnmix_v_page_bytes] u8
 *   block_table [B][max_blocks] int32: page p of sequence b is block block_table[b][p]; only
 *            the first lens[b].n_pages entries of a row are read (and the first entry of rows
 *            whose split plan starts a page there), each clamped to [0, n_blocks)
 *   the other arguments as in pnmix_decode_attn, with max_blocks in place of max_pages; the
 *   workspace is pnmix_decode_workspace_bytes(cfg, B, max_blocks) bytes.
 * Pages are written into pool blocks with pnmix_quantize_k_page / pnmix_quantize_v_page (each
 * job names its destination). */
pnmix_status pnmix_decode_attn_paged(const pnmix_cfg* cfg, int32_t B, int32_t max_blocks,
                                     const uint16_t* q, const uint16_t* k_sink,
                                     const uint16_t* v_sink, const uint8_t* k_pool,
                                     const uint8_t* v_pool, int64_t n_blocks,
                                     const int32_t* block_table, const uint16_t* k_res,
                                     const uint16_t* v_res, const pnmix_seq_len* lens,
                                     const uint32_t* mask, float sm_scale, float* out, void* ws,
                                     size_t ws_bytes, void* stream);

/* ---- analysis: dequantized pages ----------------------------------------------------------- */

/* x = S code + Z of every element of n_pages packed key pages, with the stored fp16 S and Z and
 * one fp32 fma (the exact product plus offset, rounded once) ([PNMIX] sec. 2, Eq. 2: the
 * reconstruction s q + z).  For inspection and fidelity measurement; decode never forms it.
 *   pages [n_pages][pnmix_k_page_bytes] u8 (contiguous); mask [n_pages][mask_words], the row
 *   each page was packed with; out [n_pages][N][d] f32. */
pnmix_status pnmix_dequant_k_pages(const pnmix_cfg* cfg, int32_t n_pages, const uint8_t* pages,
                                   const uint32_t* mask, float* out, void* stream);
/* The same for value pages: pages [n_pages][pnmix_v_page_bytes] u8 -> out [n_pages][N][d] f32
 * (b_V = 16 pages: the fp16 values). */
pnmix_status pnmix_dequant_v_pages(const pnmix_cfg* cfg, int32_t n_pages, const uint8_t* pages,
                                   float* out, void* stream);

/* ---- online cache placement ([PNMIX] sec. 2: new keys and values enter the FP16 residual
 * buffer of N tokens, which is quantized and appended to the cache when full; sec. 5: the
 * first N_s tokens are FP16 sinks) ------------------------------------------------------- */

/* Place one new token per sequence and advance its length on the device.
 *   k_new, v_new [B][H_kv][d] fp16; sinks, residual, lens as in pnmix_decode_attn.
 * Sequence b writes row sink_len of the sinks while sink_len < N_s and it has neither pages
 * nor residual rows (then sink_len += 1); otherwise row res_len of the residual buffer
 * (then res_len += 1).  A sequence whose residual buffer already holds N rows is left
 * unchanged (the caller must quantize it first: pnmix_quantize_*_page + pnmix_commit_page). */
pnmix_status pnmix_append_kv(const pnmix_cfg* cfg, int32_t B, const uint16_t* k_new,
                             const uint16_t* v_new, uint16_t* k_sink, uint16_t* v_sink,
                             uint16_t* k_res, uint16_t* v_res, pnmix_seq_len* lens, void* stream);

/* After the residual buffers of the batch were quantized into page slot n_pages: for every
 * sequence whose res_len == N, n_pages += 1 (up to max_pages) and res_len = 0. */
pnmix_status pnmix_commit_page(const pnmix_cfg* cfg, int32_t B, int32_t max_pages,
                               pnmix_seq_len* lens, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PNMIX_H */
