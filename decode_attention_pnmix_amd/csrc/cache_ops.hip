// cache_ops.hip -- online placement of decode tokens in the fp16 sink / residual rows.
//
// PN-Mix paper (arXiv 2610.19605) sec. 2: newly generated keys and values are kept in an FP16
// residual buffer of N tokens and quantized when it is full; sec. 5: the first N_s tokens of a
// sequence stay in FP16 as sinks.  These kernels move one token per (sequence, KV head) into
// place and keep the per-sequence lengths on the device, so a decode step needs no host
// bookkeeping between launches.
#include "common.h"
#include "kernels.h"

namespace pnmix {

// One workgroup per sequence; every thread copies 8-byte pieces of the (H_kv x d) token.
__global__ void __launch_bounds__(256) append_kv_kernel(const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new,
                                                        uint16_t* k_sink, uint16_t* v_sink,
                                                        uint16_t* k_res, uint16_t* v_res,
                                                        pnmix_seq_len* lens, int H_kv, int d,
                                                        int N_s, int N) {
  __shared__ int dst_kind;  // 0 sink, 1 residual, 2 none
  __shared__ int dst_row;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) {
    const pnmix_seq_len L = lens[b];
    if (L.sink_len < N_s && L.n_pages == 0 && L.res_len == 0) {
      dst_kind = 0;
      dst_row = max(L.sink_len, 0);
    } else if (L.res_len >= 0 && L.res_len < N) {
      dst_kind = 1;
      dst_row = L.res_len;
    } else {
      dst_kind = 2;
      dst_row = 0;
    }
  }
  __syncthreads();
  const int kind = dst_kind, row = dst_row;
  if (kind == 2) return;
  const int cap = kind == 0 ? N_s : N;
  uint16_t* kd = kind == 0 ? k_sink : k_res;
  uint16_t* vd = kind == 0 ? v_sink : v_res;
  const int per = d / 4;  // 4 fp16 per 8-byte piece
  for (int i = threadIdx.x; i < H_kv * per; i += blockDim.x) {
    const int h = i / per, c4 = i % per;
    const int64_t src = ((int64_t)b * H_kv + h) * d + c4 * 4;
    const int64_t dst = (((int64_t)b * H_kv + h) * cap + row) * d + c4 * 4;
    *reinterpret_cast<uint2*>(kd + dst) = *reinterpret_cast<const uint2*>(k_new + src);
    *reinterpret_cast<uint2*>(vd + dst) = *reinterpret_cast<const uint2*>(v_new + src);
  }
  __syncthreads();  // every thread has read lens[b] through dst_kind before it changes
  if (threadIdx.x == 0) {
    if (kind == 0)
      lens[b].sink_len = row + 1;
    else
      lens[b].res_len = row + 1;
  }
}

__global__ void commit_page_kernel(pnmix_seq_len* lens, int B, int max_pages, int N) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  pnmix_seq_len L = lens[b];
  if (L.res_len == N && L.n_pages < max_pages) {
    L.n_pages += 1;
    L.res_len = 0;
    lens[b] = L;
  }
}

hipError_t launch_append_kv(const pnmix_cfg& c, int B, const uint16_t* k_new,
                            const uint16_t* v_new, uint16_t* k_sink, uint16_t* v_sink,
                            uint16_t* k_res, uint16_t* v_res, pnmix_seq_len* lens,
                            hipStream_t stream) {
  hipLaunchKernelGGL(append_kv_kernel, dim3(B), dim3(256), 0, stream, k_new, v_new, k_sink,
                     v_sink, k_res, v_res, lens, c.H_kv, c.d, c.N_s, c.N);
  return hipGetLastError();
}

hipError_t launch_commit_page(const pnmix_cfg& c, int B, int max_pages, pnmix_seq_len* lens,
                              hipStream_t stream) {
  hipLaunchKernelGGL(commit_page_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, lens, B,
                     max_pages, c.N);
  return hipGetLastError();
}

}  // namespace pnmix
