// kernels.h -- internal launch interface between the C ABI (pnmix_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pnmix.h"

namespace pnmix {

hipError_t launch_score(const pnmix_cfg& c, int B, int P, const uint16_t* q, const uint16_t* k,
                        float* sigma, uint32_t* mask, void* ws, hipStream_t stream);
size_t score_workspace_bytes(const pnmix_cfg& c, int B, int P);
hipError_t launch_score_chunks(const pnmix_cfg& c, int B, int P, const uint16_t* q,
                               const uint16_t* k, float* chunk_sums, int skip_Ns,
                               int skip_pages, hipStream_t stream);
hipError_t launch_score_select(const pnmix_cfg& c, int B, int P, float* chunk_sums,
                               float* sigma, uint32_t* mask, hipStream_t stream);
size_t prefill_workspace_bytes(const pnmix_cfg& c, int B, int P);
hipError_t launch_prefill_fused(const pnmix_cfg& c, int B, int P, const uint16_t* q,
                                const uint16_t* k, const uint16_t* v, float* sigma,
                                uint32_t* mask, uint8_t* k_pages, uint8_t* v_pages,
                                int max_pages, void* ws, hipStream_t stream);

hipError_t launch_quantize_k(const pnmix_cfg& c, int n_pages, const pnmix_page* pages,
                             const uint32_t* mask, hipStream_t stream);
hipError_t launch_quantize_v(const pnmix_cfg& c, int n_pages, const pnmix_page* pages,
                             hipStream_t stream);
hipError_t launch_quantize_kv(const pnmix_cfg& c, int n_pages, const pnmix_page* kjobs,
                              const pnmix_page* vjobs, const uint32_t* mask, hipStream_t stream);
hipError_t launch_dequant_k(const pnmix_cfg& c, int n_pages, const uint8_t* pages,
                            const uint32_t* mask, float* out, hipStream_t stream);
hipError_t launch_dequant_v(const pnmix_cfg& c, int n_pages, const uint8_t* pages, float* out,
                            hipStream_t stream);

struct DecodePlan {
  int splits;           // partials per (sequence, KV head): workgroups of the split kernel
  int page_splits;      // waves over the packed pages, per (sequence, KV head)
  int n16;              // waves over the fp16 sink and residual rows, per (sequence, KV head)
  int fold16;           // > 0: no fp16 splits; the page splits take the fold16 32-token pieces
                        // of the fp16 rows (one wave per workgroup, n16 = 0)
  int nw;               // waves per workgroup (their partials are merged on chip)
  int pages_per_split;  // most pages of one page wave (a sequence's pages are split evenly)
  size_t ws_bytes;      // workspace for the partials
  size_t lds_wave;      // LDS slice of one wave
  size_t lds_bytes;     // dynamic LDS of one workgroup
};
bool decode_fast_path(const pnmix_cfg& c);
DecodePlan decode_plan(const pnmix_cfg& c, int B, int max_pages);
hipError_t launch_decode(const pnmix_cfg& c, int B, int max_pages, const uint16_t* q,
                         const uint16_t* k_sink, const uint16_t* v_sink, const uint8_t* k_pages,
                         const uint8_t* v_pages, const uint16_t* k_res, const uint16_t* v_res,
                         const pnmix_seq_len* lens, const uint32_t* mask, float sm_scale,
                         float* out, void* ws, hipStream_t stream,
                         const int32_t* block_table = nullptr, int64_t n_blocks = 0,
                         const uint16_t* k_new = nullptr, const uint16_t* v_new = nullptr,
                         pnmix_seq_len* lens_out = nullptr);

hipError_t launch_append_kv(const pnmix_cfg& c, int B, const uint16_t* k_new,
                            const uint16_t* v_new, uint16_t* k_sink, uint16_t* v_sink,
                            uint16_t* k_res, uint16_t* v_res, pnmix_seq_len* lens,
                            hipStream_t stream);
hipError_t launch_commit_page(const pnmix_cfg& c, int B, int max_pages, pnmix_seq_len* lens,
                              hipStream_t stream);

}  // namespace pnmix
