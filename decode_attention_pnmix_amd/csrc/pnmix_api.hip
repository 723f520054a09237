// pnmix_api.hip -- the C ABI of libpnmix.so: host-side validation, size queries and launches.
// Declarations and the contract of every entry point are in include/pnmix.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "kernels.h"
#include "pnmix.h"

// Split-K partials of pnmix_decode_attn_noalloc: a device array the library owns, one copy per
// GPU (each device that loads the library holds its own until the process ends).  Host code
// never passes this name to a kernel: it is the host-side stand-in of the symbol, and the
// device address comes from hipGetSymbolAddress (scratch_ptr below).
static constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = "";

pnmix_status fail(pnmix_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

pnmix_status ok() {
  g_err[0] = '\0';
  return PNMIX_OK;
}

pnmix_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PNMIX_E_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

pnmix_status check(const pnmix_cfg* c) {
  if (!c) return fail(PNMIX_E_INVALID, "cfg is NULL");
  if (c->H_q <= 0 || c->H_kv <= 0) return fail(PNMIX_E_INVALID, "H_q, H_kv must be positive");
  if (c->H_q % c->H_kv) return fail(PNMIX_E_INVALID, "H_q %% H_kv != 0");
  if (c->H_q / c->H_kv > 16) return fail(PNMIX_E_UNSUPPORTED, "n_g = H_q/H_kv > 16");
  if (c->d != 32 && c->d != 64 && c->d != 128)
    return fail(c->d > 0 && c->d % 2 == 0 ? PNMIX_E_UNSUPPORTED : PNMIX_E_INVALID,
                "head_dim %d not in {32, 64, 128}", c->d);
  if (c->pairing != PNMIX_PAIRS_ADJACENT && c->pairing != PNMIX_PAIRS_SPLIT_HALF)
    return fail(PNMIX_E_INVALID, "pairing %d unknown", c->pairing);
  if (c->n_hi_pairs < 0 || c->n_hi_pairs > c->d / 2)
    return fail(PNMIX_E_INVALID, "n_hi_pairs %d outside [0, d/2]", c->n_hi_pairs);
  if (c->N != 128) return fail(PNMIX_E_UNSUPPORTED, "page length N = %d (only 128)", c->N);
  if (c->G <= 0 || c->N % c->G) return fail(PNMIX_E_INVALID, "G = %d does not divide N", c->G);
  if (c->G != 32 && c->G != 64 && c->G != 128)
    return fail(PNMIX_E_UNSUPPORTED, "G = %d not in {32, 64, 128}", c->G);
  if (c->b_L < 1 || c->b_H < c->b_L || c->b_H > 8)
    return fail(PNMIX_E_INVALID, "(b_H, b_L) = (%d, %d): need 1 <= b_L <= b_H", c->b_H, c->b_L);
  if (c->b_H > 4)
    return fail(PNMIX_E_UNSUPPORTED, "(b_H, b_L) = (%d, %d): bit widths above 4", c->b_H, c->b_L);
  if (c->b_V != 1 && c->b_V != 2 && c->b_V != 4 && c->b_V != 16)
    return fail(PNMIX_E_UNSUPPORTED, "b_V = %d not in {1, 2, 4, 16}", c->b_V);
  if (c->g_V <= 0 || c->d % c->g_V) return fail(PNMIX_E_INVALID, "g_V = %d does not divide d", c->g_V);
  if (c->g_V != 16 && c->g_V != 32 && c->g_V != 64 && c->g_V != 128)
    return fail(PNMIX_E_UNSUPPORTED, "g_V = %d not in {16, 32, 64, 128}", c->g_V);
  if (c->d / c->g_V > 4)
    return fail(PNMIX_E_UNSUPPORTED, "d / g_V = %d value groups per token (at most 4)", c->d / c->g_V);
  if (c->N_s < 0 || c->N_s > 128) return fail(PNMIX_E_INVALID, "N_s = %d outside [0, 128]", c->N_s);
  return PNMIX_OK;
}

}  // namespace

extern "C" {

pnmix_status pnmix_check_cfg(const pnmix_cfg* cfg) {
  const pnmix_status s = check(cfg);
  return s == PNMIX_OK ? ok() : s;
}

int32_t pnmix_hi_pairs(double r, int32_t d) {
  if (!(r >= 0.0) || d <= 0) return 0;
  if (r > 1.0) r = 1.0;
  return (int32_t)std::floor(r * (double)(d / 2) + 1e-9);
}

size_t pnmix_mask_words(const pnmix_cfg* c) { return c ? (size_t)(c->d / 2 + 31) / 32 : 0; }

size_t pnmix_k_page_bytes(const pnmix_cfg* c) {
  if (!c || c->G <= 0 || c->b_L < 0 || c->b_H < c->b_L) return 0;
  return (size_t)c->N * c->d * c->b_L / 8 +
         (size_t)c->N * 2 * c->n_hi_pairs * (c->b_H - c->b_L) / 8 +
         4 * (size_t)(c->N / c->G) * c->d;
}

size_t pnmix_v_page_bytes(const pnmix_cfg* c) {
  if (!c || c->g_V <= 0 || c->b_V <= 0) return 0;
  if (c->b_V == 16) return 2 * (size_t)c->N * c->d;
  return (size_t)c->N * c->d * c->b_V / 8 + 4 * (size_t)c->N * (c->d / c->g_V);
}

size_t pnmix_score_workspace_bytes(const pnmix_cfg* c, int32_t B, int32_t P) {
  if (check(c) != PNMIX_OK || B <= 0 || P <= 0) return 0;
  return pnmix::score_workspace_bytes(*c, B, P);
}

int32_t pnmix_decode_splits(const pnmix_cfg* c, int32_t B, int32_t max_pages) {
  if (check(c) != PNMIX_OK || B <= 0 || max_pages < 0) return 0;
  return pnmix::decode_plan(*c, B, max_pages).splits;
}

pnmix_status pnmix_decode_plan(const pnmix_cfg* c, int32_t B, int32_t max_pages, int32_t* out) {
  const pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (B <= 0 || max_pages < 0 || !out)
    return fail(PNMIX_E_INVALID, "decode plan: B > 0, max_pages >= 0 and out needed");
  const pnmix::DecodePlan p = pnmix::decode_plan(*c, B, max_pages);
  out[0] = p.splits;
  out[1] = p.page_splits;
  out[2] = p.n16;
  out[3] = p.nw;
  return PNMIX_OK;
}

size_t pnmix_decode_workspace_bytes(const pnmix_cfg* c, int32_t B, int32_t max_pages) {
  if (check(c) != PNMIX_OK || B <= 0 || max_pages < 0) return 0;
  return pnmix::decode_plan(*c, B, max_pages).ws_bytes;
}

const char* pnmix_last_error(void) { return g_err; }

pnmix_status pnmix_score_prefill(const pnmix_cfg* c, int32_t B, int32_t P, const uint16_t* q,
                                 const uint16_t* k, float* sigma, uint32_t* mask, void* ws,
                                 size_t ws_bytes, void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (B <= 0 || P <= 0) return fail(PNMIX_E_INVALID, "B = %d, P = %d must be positive", B, P);
  if ((long long)B * (c->H_q + c->H_kv) > 0x7FFFFFFFLL || (P + 63) / 64 > 65535)
    return fail(PNMIX_E_UNSUPPORTED, "B * (H_q + H_kv) >= 2^31 or P > 65535 * 64");
  if (!q || !k || !mask || !ws) return fail(PNMIX_E_INVALID, "q, k, mask and ws must be non-NULL");
  if (ws_bytes < pnmix::score_workspace_bytes(*c, B, P))
    return fail(PNMIX_E_WORKSPACE, "score workspace %zu < %zu bytes", ws_bytes,
                pnmix::score_workspace_bytes(*c, B, P));
  return hip_status(pnmix::launch_score(*c, B, P, q, k, sigma, mask, ws, (hipStream_t)stream),
                    "pnmix_score_prefill");
}

size_t pnmix_prefill_fused_workspace_bytes(const pnmix_cfg* c, int32_t B, int32_t P) {
  if (check(c) != PNMIX_OK || B <= 0 || P <= 0) return 0;
  return pnmix::prefill_workspace_bytes(*c, B, P);
}

pnmix_status pnmix_prefill_fused(const pnmix_cfg* c, int32_t B, int32_t P, const uint16_t* q,
                                 const uint16_t* k, const uint16_t* v, float* sigma,
                                 uint32_t* mask, uint8_t* k_pages, uint8_t* v_pages,
                                 int32_t max_pages, void* ws, size_t ws_bytes, void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (c->b_H != 3 || c->b_L != 1 || c->b_V != 2)
    return fail(PNMIX_E_UNSUPPORTED,
                "fused prefill serves (b_H, b_L, b_V) = (3, 1, 2); for other widths call "
                "pnmix_score_prefill and pnmix_quantize_kv_pages");
  if (B <= 0 || P <= 0 || max_pages < 0)
    return fail(PNMIX_E_INVALID, "B = %d, P = %d must be positive, max_pages = %d >= 0", B, P,
                max_pages);
  if ((long long)B * (c->H_q + c->H_kv) > 0x7FFFFFFFLL || (P + 63) / 64 > 65535)
    return fail(PNMIX_E_UNSUPPORTED, "B * (H_q + H_kv) >= 2^31 or P > 65535 * 64");
  const int n_full = P > c->N_s ? (P - c->N_s) / c->N : 0;
  if (n_full > max_pages)
    return fail(PNMIX_E_INVALID, "the prompt fills %d pages, max_pages = %d", n_full, max_pages);
  if (!q || !k || !v || !mask || !ws || (n_full > 0 && (!k_pages || !v_pages)))
    return fail(PNMIX_E_INVALID, "q, k, v, mask, ws (and the page arrays) must be non-NULL");
  const size_t need = pnmix::prefill_workspace_bytes(*c, B, P);
  if (ws_bytes < need)
    return fail(PNMIX_E_WORKSPACE, "fused prefill workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(pnmix::launch_prefill_fused(*c, B, P, q, k, v, sigma, mask, k_pages, v_pages,
                                                max_pages, ws, (hipStream_t)stream),
                    "pnmix_prefill_fused");
}

pnmix_status pnmix_quantize_k_page(const pnmix_cfg* c, int32_t n_pages, const pnmix_page* pages,
                                   const uint32_t* mask, void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (n_pages < 0) return fail(PNMIX_E_INVALID, "n_pages = %d < 0", n_pages);
  if (n_pages == 0) return ok();
  if (!pages || !mask) return fail(PNMIX_E_INVALID, "pages and mask must be non-NULL");
  return hip_status(pnmix::launch_quantize_k(*c, n_pages, pages, mask, (hipStream_t)stream),
                    "pnmix_quantize_k_page");
}

pnmix_status pnmix_quantize_v_page(const pnmix_cfg* c, int32_t n_pages, const pnmix_page* pages,
                                   void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (n_pages < 0) return fail(PNMIX_E_INVALID, "n_pages = %d < 0", n_pages);
  if (n_pages == 0) return ok();
  if (!pages) return fail(PNMIX_E_INVALID, "pages must be non-NULL");
  return hip_status(pnmix::launch_quantize_v(*c, n_pages, pages, (hipStream_t)stream),
                    "pnmix_quantize_v_page");
}

pnmix_status pnmix_quantize_kv_pages(const pnmix_cfg* c, int32_t n_pages,
                                     const pnmix_page* k_pages, const pnmix_page* v_pages,
                                     const uint32_t* mask, void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (n_pages < 0) return fail(PNMIX_E_INVALID, "n_pages = %d < 0", n_pages);
  if (n_pages == 0) return ok();
  if (!k_pages || !v_pages || !mask)
    return fail(PNMIX_E_INVALID, "k_pages, v_pages and mask must be non-NULL");
  return hip_status(pnmix::launch_quantize_kv(*c, n_pages, k_pages, v_pages, mask,
                                              (hipStream_t)stream),
                    "pnmix_quantize_kv_pages");
}

// Argument checks shared by the contiguous decode entry points (before any HIP call).
static pnmix_status check_decode(const pnmix_cfg* c, int32_t B, int32_t max_pages,
                                 const uint16_t* q, const uint16_t* k_sink,
                                 const uint16_t* v_sink, const uint8_t* k_pages,
                                 const uint8_t* v_pages, const uint16_t* k_res,
                                 const uint16_t* v_res, const pnmix_seq_len* lens,
                                 const uint32_t* mask, float sm_scale, float* out, void* ws,
                                 size_t ws_bytes) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (B <= 0 || max_pages < 0)
    return fail(PNMIX_E_INVALID, "B = %d must be positive, max_pages = %d >= 0", B, max_pages);
  if ((long long)B * c->H_kv > 65535) return fail(PNMIX_E_UNSUPPORTED, "B * H_kv > 65535");
  if (!q || !k_res || !v_res || !lens || !mask || !out || !ws)
    return fail(PNMIX_E_INVALID, "q, k_res, v_res, lens, mask, out and ws must be non-NULL");
  if (c->N_s > 0 && (!k_sink || !v_sink))
    return fail(PNMIX_E_INVALID, "k_sink and v_sink must be non-NULL when N_s > 0");
  if (max_pages > 0 && (!k_pages || !v_pages))
    return fail(PNMIX_E_INVALID, "k_pages and v_pages must be non-NULL when max_pages > 0");
  if ((long long)max_pages * c->H_kv *
          (long long)std::max(pnmix_k_page_bytes(c), pnmix_v_page_bytes(c)) > 0x7FFFFFFFLL)
    return fail(PNMIX_E_UNSUPPORTED,
                "max_pages * H_kv * page bytes exceeds 2 GiB (use pnmix_decode_attn_paged)");
  if (!std::isfinite(sm_scale)) return fail(PNMIX_E_INVALID, "sm_scale is not finite");
  const pnmix::DecodePlan plan = pnmix::decode_plan(*c, B, max_pages);
  if (plan.lds_wave > 65536)
    return fail(PNMIX_E_UNSUPPORTED, "n_g = %d with G = %d needs %zu bytes of LDS (> 64 KiB)",
                c->H_q / c->H_kv, c->G, plan.lds_wave);
  if (ws_bytes < plan.ws_bytes)
    return fail(PNMIX_E_WORKSPACE, "decode workspace %zu < %zu bytes", ws_bytes, plan.ws_bytes);
  return PNMIX_OK;
}

pnmix_status pnmix_decode_attn(const pnmix_cfg* c, int32_t B, int32_t max_pages,
                               const uint16_t* q, const uint16_t* k_sink, const uint16_t* v_sink,
                               const uint8_t* k_pages, const uint8_t* v_pages,
                               const uint16_t* k_res, const uint16_t* v_res,
                               const pnmix_seq_len* lens, const uint32_t* mask, float sm_scale,
                               float* out, void* ws, size_t ws_bytes, void* stream) {
  const pnmix_status s = check_decode(c, B, max_pages, q, k_sink, v_sink, k_pages, v_pages,
                                      k_res, v_res, lens, mask, sm_scale, out, ws, ws_bytes);
  if (s != PNMIX_OK) return s;
  return hip_status(pnmix::launch_decode(*c, B, max_pages, q, k_sink, v_sink, k_pages, v_pages,
                                         k_res, v_res, lens, mask, sm_scale, out, ws,
                                         (hipStream_t)stream),
                    "pnmix_decode_attn");
}

pnmix_status pnmix_append_decode_attn(const pnmix_cfg* c, int32_t B, int32_t max_pages,
                                      const uint16_t* q, const uint16_t* k_new,
                                      const uint16_t* v_new, uint16_t* k_sink, uint16_t* v_sink,
                                      const uint8_t* k_pages, const uint8_t* v_pages,
                                      uint16_t* k_res, uint16_t* v_res,
                                      const pnmix_seq_len* lens, pnmix_seq_len* lens_out,
                                      const uint32_t* mask, float sm_scale, float* out, void* ws,
                                      size_t ws_bytes, void* stream) {
  const pnmix_status s = check_decode(c, B, max_pages, q, k_sink, v_sink, k_pages, v_pages,
                                      k_res, v_res, lens, mask, sm_scale, out, ws, ws_bytes);
  if (s != PNMIX_OK) return s;
  if (!k_new || !v_new || !lens_out)
    return fail(PNMIX_E_INVALID, "k_new, v_new and lens_out must be non-NULL");
  const char* lo = reinterpret_cast<const char*>(lens_out);
  const char* li = reinterpret_cast<const char*>(lens);
  const size_t lb = (size_t)B * sizeof(pnmix_seq_len);
  if (lo < li + lb && li < lo + lb)
    return fail(PNMIX_E_INVALID, "lens_out must not overlap lens");
  return hip_status(pnmix::launch_decode(*c, B, max_pages, q, k_sink, v_sink, k_pages, v_pages,
                                         k_res, v_res, lens, mask, sm_scale, out, ws,
                                         (hipStream_t)stream, nullptr, 0, k_new, v_new, lens_out),
                    "pnmix_append_decode_attn");
}

// Device address of this GPU's scratch array, looked up once per device with that device
// current (the first call on the device; later calls reuse it).
static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static pnmix_status scratch_ptr(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "pnmix_decode_attn_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PNMIX_E_UNSUPPORTED, "pnmix_decode_attn_noalloc: device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t s = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (s != hipSuccess || !ptr)
      return hip_status(s != hipSuccess ? s : hipErrorInvalidSymbol,
                        "pnmix_decode_attn_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PNMIX_OK;
}

size_t pnmix_noalloc_scratch_bytes(void) { return kScratchBytes; }

pnmix_status pnmix_decode_attn_noalloc(const pnmix_cfg* c, int32_t B, int32_t max_pages,
                                       const uint16_t* q, const uint16_t* k_sink,
                                       const uint16_t* v_sink, const uint8_t* k_pages,
                                       const uint8_t* v_pages, const uint16_t* k_res,
                                       const uint16_t* v_res, const pnmix_seq_len* lens,
                                       const uint32_t* mask, float sm_scale, float* out,
                                       void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (B <= 0 || max_pages < 0)
    return fail(PNMIX_E_INVALID, "B = %d must be positive, max_pages = %d >= 0", B, max_pages);
  const size_t need = pnmix::decode_plan(*c, B, max_pages).ws_bytes;
  if (need > kScratchBytes)
    return fail(PNMIX_E_WORKSPACE,
                "pnmix_decode_attn_noalloc: B = %d, max_pages = %d need %zu bytes of split-K "
                "partials, more than the library's %zu-byte scratch (use pnmix_decode_attn with "
                "a workspace)", B, max_pages, need, kScratchBytes);
  // the fake workspace pointer only passes the NULL check; the real one replaces it below
  s = check_decode(c, B, max_pages, q, k_sink, v_sink, k_pages, v_pages, k_res, v_res, lens, mask,
                   sm_scale, out, reinterpret_cast<void*>(static_cast<uintptr_t>(256)),
                   kScratchBytes);
  if (s != PNMIX_OK) return s;
  void* ws = nullptr;
  s = scratch_ptr(&ws);
  if (s != PNMIX_OK) return s;
  return hip_status(pnmix::launch_decode(*c, B, max_pages, q, k_sink, v_sink, k_pages, v_pages,
                                         k_res, v_res, lens, mask, sm_scale, out, ws,
                                         (hipStream_t)stream),
                    "pnmix_decode_attn_noalloc");
}

pnmix_status pnmix_decode_attn_paged(const pnmix_cfg* c, int32_t B, int32_t max_blocks,
                                     const uint16_t* q, const uint16_t* k_sink,
                                     const uint16_t* v_sink, const uint8_t* k_pool,
                                     const uint8_t* v_pool, int64_t n_blocks,
                                     const int32_t* block_table, const uint16_t* k_res,
                                     const uint16_t* v_res, const pnmix_seq_len* lens,
                                     const uint32_t* mask, float sm_scale, float* out, void* ws,
                                     size_t ws_bytes, void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (B <= 0 || max_blocks < 0)
    return fail(PNMIX_E_INVALID, "B = %d must be positive, max_blocks = %d >= 0", B, max_blocks);
  if ((long long)B * c->H_kv > 65535) return fail(PNMIX_E_UNSUPPORTED, "B * H_kv > 65535");
  if (!q || !k_res || !v_res || !lens || !mask || !out || !ws)
    return fail(PNMIX_E_INVALID, "q, k_res, v_res, lens, mask, out and ws must be non-NULL");
  if (c->N_s > 0 && (!k_sink || !v_sink))
    return fail(PNMIX_E_INVALID, "k_sink and v_sink must be non-NULL when N_s > 0");
  if (max_blocks > 0 && (!k_pool || !v_pool || !block_table || n_blocks <= 0))
    return fail(PNMIX_E_INVALID,
                "k_pool, v_pool and block_table must be non-NULL and n_blocks > 0 when "
                "max_blocks > 0");
  if (!std::isfinite(sm_scale)) return fail(PNMIX_E_INVALID, "sm_scale is not finite");
  const pnmix::DecodePlan plan = pnmix::decode_plan(*c, B, max_blocks);
  if (plan.lds_wave > 65536)
    return fail(PNMIX_E_UNSUPPORTED, "n_g = %d with G = %d needs %zu bytes of LDS (> 64 KiB)",
                c->H_q / c->H_kv, c->G, plan.lds_wave);
  if (ws_bytes < plan.ws_bytes)
    return fail(PNMIX_E_WORKSPACE, "decode workspace %zu < %zu bytes", ws_bytes, plan.ws_bytes);
  return hip_status(pnmix::launch_decode(*c, B, max_blocks, q, k_sink, v_sink, k_pool, v_pool,
                                         k_res, v_res, lens, mask, sm_scale, out, ws,
                                         (hipStream_t)stream, max_blocks > 0 ? block_table : nullptr,
                                         n_blocks),
                    "pnmix_decode_attn_paged");
}

pnmix_status pnmix_dequant_k_pages(const pnmix_cfg* c, int32_t n_pages, const uint8_t* pages,
                                   const uint32_t* mask, float* out, void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (n_pages < 0) return fail(PNMIX_E_INVALID, "n_pages = %d < 0", n_pages);
  if (n_pages == 0) return ok();
  if (!pages || !mask || !out) return fail(PNMIX_E_INVALID, "pages, mask and out must be non-NULL");
  return hip_status(pnmix::launch_dequant_k(*c, n_pages, pages, mask, out, (hipStream_t)stream),
                    "pnmix_dequant_k_pages");
}

pnmix_status pnmix_dequant_v_pages(const pnmix_cfg* c, int32_t n_pages, const uint8_t* pages,
                                   float* out, void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (n_pages < 0) return fail(PNMIX_E_INVALID, "n_pages = %d < 0", n_pages);
  if (n_pages == 0) return ok();
  if (!pages || !out) return fail(PNMIX_E_INVALID, "pages and out must be non-NULL");
  return hip_status(pnmix::launch_dequant_v(*c, n_pages, pages, out, (hipStream_t)stream),
                    "pnmix_dequant_v_pages");
}

pnmix_status pnmix_append_kv(const pnmix_cfg* c, int32_t B, const uint16_t* k_new,
                             const uint16_t* v_new, uint16_t* k_sink, uint16_t* v_sink,
                             uint16_t* k_res, uint16_t* v_res, pnmix_seq_len* lens,
                             void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (B <= 0) return fail(PNMIX_E_INVALID, "B = %d must be positive", B);
  if (!k_new || !v_new || !k_res || !v_res || !lens)
    return fail(PNMIX_E_INVALID, "k_new, v_new, k_res, v_res and lens must be non-NULL");
  if (c->N_s > 0 && (!k_sink || !v_sink))
    return fail(PNMIX_E_INVALID, "k_sink and v_sink must be non-NULL when N_s > 0");
  return hip_status(pnmix::launch_append_kv(*c, B, k_new, v_new, k_sink, v_sink, k_res, v_res,
                                            lens, (hipStream_t)stream),
                    "pnmix_append_kv");
}

pnmix_status pnmix_commit_page(const pnmix_cfg* c, int32_t B, int32_t max_pages,
                               pnmix_seq_len* lens, void* stream) {
  pnmix_status s = check(c);
  if (s != PNMIX_OK) return s;
  if (B <= 0 || max_pages < 0 || !lens)
    return fail(PNMIX_E_INVALID, "B > 0, max_pages >= 0 and lens non-NULL required");
  return hip_status(pnmix::launch_commit_page(*c, B, max_pages, lens, (hipStream_t)stream),
                    "pnmix_commit_page");
}

}  // extern "C"
