// score.hip -- Eq. 6 prefill pair-norm saliency and the fixed pair mask on gfx950.
//
// "PN-Mix: Key-Cache Precision Allocation from RoPE Channel-Pair Norms", Core equations, Eq. 6:
// sigma_{h,i} = (1/n_g) sum_{h' in g^-1(h)} E_t||q_{h',t,i}|| * E_s||k_{h,s,i}||, then the top
// floor(r d/2) pairs of each KV head form a bit mask stored once (Korean summary page,
// "무엇과 다른가": B x L x H_kv x d/2 bits).
//
// Two passes.  Pass 1 gives each (sequence, head, 64-token chunk) one wave; the wave stages 32
// token rows at a time in LDS with 16-byte loads, and lane i owns RoPE pair i and adds its pair
// norms over the chunk in ascending token order.  Pass 2 gives each (sequence, KV head) one
// workgroup: its waves add the chunk sums of one head each in ascending chunk order (the loads
// go out 32 chunks at a time), divide by P, then wave 0 forms sigma, ranks the pairs through
// LDS and writes the mask with a wave ballot.  The summation order is fixed, so sigma and the
// mask are bit-identical to the reference oracle.
#include "common.h"
#include "kernels.h"

namespace pnmix {

constexpr int kChunk = 64;

constexpr int kSub = 32;  // tokens staged in LDS at a time

// Key chunks cover_lo..cover_hi are skipped when the caller computes them elsewhere (the fused
// prefill's page workgroups); cover_lo > cover_hi skips none.
__global__ void __launch_bounds__(64) score_chunks_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          float* __restrict__ chunk_sums,
                                                          int H_q, int H_kv, int d, int pairing,
                                                          int P, int n_chunks, int cover_lo,
                                                          int cover_hi) {
  __shared__ __align__(16) uint16_t tile[kSub * 128];  // kSub token rows of up to 128 fp16
  const int seq_head = blockIdx.x;  // b * (H_q + H_kv) + head (grid x: no 65535 limit)
  const int chunk = blockIdx.y;
  const int H = H_q + H_kv;
  const int b = seq_head / H;
  const int head = seq_head % H;
  if (head >= H_q && chunk >= cover_lo && chunk <= cover_hi) return;  // whole workgroup
  const int np = d / 2;
  const int i = threadIdx.x;
  const uint16_t* src = head < H_q ? q + ((int64_t)b * H_q + head) * P * d
                                   : k + ((int64_t)b * H_kv + (head - H_q)) * P * d;
  const int c0 = pairing == PNMIX_PAIRS_ADJACENT ? 2 * i : i;
  const int c1 = pairing == PNMIX_PAIRS_ADJACENT ? 2 * i + 1 : i + np;
  const int t0 = chunk * kChunk;
  const int t1 = min(t0 + kChunk, P);
  // The wave copies kSub token rows at a time into LDS with 16-byte loads (the rows of a
  // (sequence, head) are contiguous; d * 2 bytes is a multiple of 16), or with 2-byte loads when
  // the rows are not 16-byte aligned; then lane i adds the norms of pair i over those tokens in
  // ascending order, as before.
  const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  float s = 0.0f;
  for (int ts = t0; ts < t1; ts += kSub) {
    const int rows = min(kSub, t1 - ts);
    const uint16_t* g = src + (int64_t)ts * d;
    if (vec) {
      const int n16 = rows * d / 8;
      for (int x = i; x < n16; x += 64)
        reinterpret_cast<uint4*>(tile)[x] = reinterpret_cast<const uint4*>(g)[x];
    } else {
      for (int x = i; x < rows * d; x += 64) tile[x] = g[x];
    }
    __syncthreads();
    if (i < np) {
#pragma unroll 8
      for (int t = 0; t < rows; ++t) {
        const float x = h2f(tile[t * d + c0]);
        const float y = h2f(tile[t * d + c1]);
        const float a = x * x;
        const float bb = y * y;
        s = s + sqrtf(a + bb);
      }
    }
    __syncthreads();  // the tile is refilled
  }
  if (i < np) chunk_sums[((int64_t)seq_head * n_chunks + chunk) * np + i] = s;
}

__global__ void __launch_bounds__(256) score_select_kernel(const float* __restrict__ chunk_sums,
                                                           float* __restrict__ sigma,
                                                           uint32_t* __restrict__ mask, int H_q,
                                                           int H_kv, int d, int P, int n_chunks,
                                                           int n_hi, int words) {
  __shared__ float means[17][64];  // n_g query heads (<= 16) then the KV head
  __shared__ float sig[64];
  const int seq = blockIdx.x / H_kv;
  const int h = blockIdx.x % H_kv;
  const int ng = H_q / H_kv;
  const int np = d / 2;
  const int H = H_q + H_kv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  for (int r = wave; r <= ng; r += nwaves) {
    const int head = r < ng ? h * ng + r : H_q + h;
    if (lane < np) {
      const float* cs = chunk_sums + ((int64_t)(seq * H + head) * n_chunks) * np + lane;
      // the adds stay in ascending chunk order; the loads go out 32 at a time
      float s = 0.0f;
      for (int c0 = 0; c0 < n_chunks; c0 += 32) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = c0 + j < n_chunks ? cs[(int64_t)(c0 + j) * np] : 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (c0 + j < n_chunks) s = s + v[j];
      }
      means[r][lane] = s / (float)P;
    }
  }
  __syncthreads();
  float sg = 0.0f;
  if (wave == 0 && lane < np) {
    float a = 0.0f;
    for (int r = 0; r < ng; ++r) a = a + means[r][lane];
    sg = (a / (float)ng) * means[ng][lane];
    sig[lane] = sg;
    if (sigma) sigma[((int64_t)seq * H_kv + h) * np + lane] = sg;
  }
  __syncthreads();
  if (wave != 0) return;
  int rank = 0;
  if (lane < np) {
    for (int j = 0; j < np; ++j) {
      const float o = sig[j];
      rank += (o > sg || (o == sg && j < lane)) ? 1 : 0;
    }
  }
  const unsigned long long bits = __ballot(lane < np && rank < n_hi);
  if (lane < words) {
    mask[((int64_t)seq * H_kv + h) * words + lane] = (uint32_t)(bits >> (32 * lane));
  }
}

hipError_t launch_score_chunks(const pnmix_cfg& c, int B, int P, const uint16_t* q,
                               const uint16_t* k, float* chunk_sums, int cover_lo, int cover_hi,
                               hipStream_t stream) {
  const int n_chunks = (P + kChunk - 1) / kChunk;
  dim3 g1(B * (c.H_q + c.H_kv), n_chunks);
  hipLaunchKernelGGL(score_chunks_kernel, g1, dim3(64), 0, stream, q, k, chunk_sums, c.H_q,
                     c.H_kv, c.d, c.pairing, P, n_chunks, cover_lo, cover_hi);
  return hipGetLastError();
}

hipError_t launch_score_select(const pnmix_cfg& c, int B, int P, const float* chunk_sums,
                               float* sigma, uint32_t* mask, hipStream_t stream) {
  const int n_chunks = (P + kChunk - 1) / kChunk;
  const int words = (c.d / 2 + 31) / 32;
  hipLaunchKernelGGL(score_select_kernel, dim3(B * c.H_kv), dim3(256), 0, stream, chunk_sums,
                     sigma, mask, c.H_q, c.H_kv, c.d, P, n_chunks, c.n_hi_pairs, words);
  return hipGetLastError();
}

hipError_t launch_score(const pnmix_cfg& c, int B, int P, const uint16_t* q, const uint16_t* k,
                        float* sigma, uint32_t* mask, void* ws, hipStream_t stream) {
  float* chunk_sums = static_cast<float*>(ws);
  const hipError_t e = launch_score_chunks(c, B, P, q, k, chunk_sums, 1, 0, stream);
  return e != hipSuccess ? e : launch_score_select(c, B, P, chunk_sums, sigma, mask, stream);
}

size_t score_workspace_bytes(const pnmix_cfg& c, int B, int P) {
  const size_t n_chunks = (size_t)(P + kChunk - 1) / kChunk;
  const size_t bytes = (size_t)B * (c.H_q + c.H_kv) * n_chunks * (c.d / 2) * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

}  // namespace pnmix
