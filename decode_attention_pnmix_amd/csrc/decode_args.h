// decode_args.h -- arguments of the decode kernels (split kernels and merge kernel) and the
// placement rule of a fused append, shared by decode.hip and decode_generic.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "pnmix.h"

namespace pnmix {


struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_sink;
  const uint16_t* v_sink;
  const uint8_t* k_pages;  // [B][max_pages][H_kv][kpb], or with a block table the pool
  const uint8_t* v_pages;  // [n_blocks][H_kv][kpb] (likewise vpb)
  const int32_t* table;    // NULL (contiguous pages) or the block table [B][max_pages]
  int64_t n_blocks;        // blocks in the pools (block table only)
  const uint16_t* k_res;
  const uint16_t* v_res;
  const pnmix_seq_len* lens;
  const uint32_t* mask;
  // Append fused into the call (NULL k_new: none): the new key and value rows [B][H_kv][d] take
  // part in the attention straight from k_new / v_new, and the merge kernel then writes them
  // into the sink or residual rows (k_sink ... v_res are the caller's writable buffers) and
  // the advanced lengths into lens_out (never the lens array every wave reads).
  const uint16_t* k_new;
  const uint16_t* v_new;
  pnmix_seq_len* lens_out;
  float* part_o;   // [B*H_kv][splits][n_g][d]
  float* part_ml;  // [B*H_kv][splits][n_g][2]
  float* out;      // [B][H_q][d]
  float qscale;    // sm_scale * log2(e)
  int H_q, H_kv, n_g, pairing, n_hi, n_sal, G, KG, g_V, NGV, N_s, max_pages, words;
  int b_H, b_L, b_V;  // bit widths (the matrix-core kernel serves (3, 1, 2))
  int64_t kpb, vpb;
  int splits;      // partials per (sequence, KV head): workgroups of the split kernel
  int page_splits; // page splits per (sequence, KV head), then n16 fp16-row splits (32-token
                   // pieces strided by n16)
  int n16;
  int fold16;      // > 0: fp16 piece i goes to page split page_splits - 1 - i (mod page_splits), nw = 1
  int nw;          // waves per workgroup, one split each
  int lds_T;       // bytes of the q.K digit table (KG * NT * 16 rows * TL)
  int lds_wave;    // LDS bytes of one wave's slice
};

// Where a fused append puts sequence b's new row, from its lengths before the call (the rule
// of the append entry point): sink row sink_len while the sinks are filling and the sequence
// has neither pages nor residual rows (kind 0), else residual row res_len if that is below N
// (kind 1), else nowhere (kind 2).
__device__ __forceinline__ void append_slot(const pnmix_seq_len& L, int N_s, int& kind, int& row) {
  if (L.sink_len < N_s && L.n_pages == 0 && L.res_len == 0) {
    kind = 0;
    row = max(L.sink_len, 0);
  } else if (L.res_len >= 0 && L.res_len < kN) {
    kind = 1;
    row = L.res_len;
  } else {
    kind = 2;
    row = 0;
  }
}


// Generic split kernel (any supported bit widths and value groups): launched by launch_decode
// when the matrix-core kernel does not serve the configuration.  Grid (splits, B * H_kv), 256
// threads, lds bytes of dynamic LDS.
hipError_t launch_generic_split(const DecodeArgs& a, int d, int B, size_t lds, hipStream_t stream);
size_t generic_lds_bytes(const pnmix_cfg& c);
// Workgroups of the generic split kernel that c selects, resident per compute unit with lds
// bytes of dynamic LDS (at least 1).
int generic_blocks_per_cu(const pnmix_cfg& c, size_t lds);

}  // namespace pnmix
