// score.hip -- Eq. 6 prefill pair-norm saliency and the fixed pair mask on gfx950.
//
// "PN-Mix: Key-Cache Precision Allocation from RoPE Channel-Pair Norms", Core equations, Eq. 6:
// sigma_{h,i} = (1/n_g) sum_{h' in g^-1(h)} E_t||q_{h',t,i}|| * E_s||k_{h,s,i}||, then the top
// floor(r d/2) pairs of each KV head form a bit mask stored once (Korean summary page,
// "무엇과 다른가": B x L x H_kv x d/2 bits).
//
// Two passes.  Pass 1 gives each (sequence, head, 64-token chunk) one wave; the wave stages the
// chunk's token rows in LDS with 16-byte loads all in flight at once, and lane i owns RoPE pair
// i and adds its pair norms over the chunk in ascending token order.  Pass 2 gives each (sequence, KV head) one
// workgroup: its waves add the chunk sums of one head each in ascending chunk order (the loads
// go out 32 chunks at a time, the next 32 in flight during the adds; for long prompts a
// workgroup per (sequence, head) adds them first, through LDS), divide by P, then wave 0 forms sigma, ranks the pairs through
// LDS and writes the mask with a wave ballot.  The summation order is fixed, so sigma and the
// mask are bit-identical to the reference oracle.
#include "common.h"
#include "kernels.h"

namespace pnmix {

constexpr int kChunk = 64;

// Key chunks that lie wholly inside one of the first skip_pages pages of N tokens after skip_Ns
// sinks are skipped: the fused prefill's page workgroups add them up (skip_pages = 0 skips
// none).  D is the head dim (row offsets in the LDS tile are then immediates).
template <int D>
__global__ void __launch_bounds__(64) score_chunks_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          float* __restrict__ chunk_sums,
                                                          int H_q, int H_kv, int pairing,
                                                          int P, int n_chunks, int skip_Ns,
                                                          int skip_pages) {
  __shared__ __align__(16) uint16_t tile[kChunk * D];  // the chunk's token rows
  const int seq_head = blockIdx.x;  // b * (H_q + H_kv) + head (grid x: no 65535 limit)
  const int chunk = blockIdx.y;
  const int H = H_q + H_kv;
  const int b = seq_head / H;
  const int head = seq_head % H;
  if (head >= H_q && skip_pages > 0) {  // whole workgroup
    const int u = chunk * kChunk - skip_Ns;
    if (u >= 0 && u + kChunk <= kN * skip_pages && (u % kN) + kChunk <= kN) return;
  }
  constexpr int np = D / 2;
  constexpr int kLoads = kChunk * D / 8 / 64;  // 16-byte loads per lane for a full chunk
  const int i = threadIdx.x;
  const uint16_t* src = head < H_q ? q + ((int64_t)b * H_q + head) * P * D
                                   : k + ((int64_t)b * H_kv + (head - H_q)) * P * D;
  const int c0 = pairing == PNMIX_PAIRS_ADJACENT ? 2 * i : i;
  const int c1 = pairing == PNMIX_PAIRS_ADJACENT ? 2 * i + 1 : i + np;
  const int t0 = chunk * kChunk;
  const int rows = min(kChunk, P - t0);
  const uint16_t* g = src + (int64_t)t0 * D;
  // The chunk's rows go to LDS: a full chunk of 16-byte-aligned rows (the rows of a (sequence,
  // head) are contiguous; D * 2 bytes is a multiple of 16) in one round, every load issued
  // before the first store; the last, partial chunk of a prompt with 16-byte loads in a loop;
  // unaligned rows element by element.  Then lane i adds the
  // norms of pair i over the chunk's tokens in ascending order.
  if (rows == kChunk && (reinterpret_cast<uintptr_t>(g) & 15) == 0) {
    uint4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) v[j] = reinterpret_cast<const uint4*>(g)[i + 64 * j];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) reinterpret_cast<uint4*>(tile)[i + 64 * j] = v[j];
  } else if ((reinterpret_cast<uintptr_t>(g) & 15) == 0) {
    for (int x = i; x < rows * D / 8; x += 64)
      reinterpret_cast<uint4*>(tile)[x] = reinterpret_cast<const uint4*>(g)[x];
  } else {
    for (int x = i; x < rows * D; x += 64) tile[x] = g[x];
  }
  __syncthreads();
  float s = 0.0f;
  if (i < np) {
    if (rows == kChunk) {
#pragma unroll 8
      for (int t = 0; t < kChunk; ++t) s = s + pair_norm(tile[t * D + c0], tile[t * D + c1]);
    } else {
      for (int t = 0; t < rows; ++t) s = s + pair_norm(tile[t * D + c0], tile[t * D + c1]);
    }
    chunk_sums[((int64_t)seq_head * n_chunks + chunk) * np + i] = s;
  }
}

constexpr int kSelLoads = 32;  // chunk-sum loads in flight per lane

// Long prompts: one workgroup of 16 waves per (sequence, head) adds that head's chunk sums.
// The chunk sums go to LDS kRowBlk chunks at a time (each wave loads kRowBlk / 16 of them, all
// in flight at once); wave 0 adds them in ascending chunk order while the waves load the next
// block into the other buffer.  The mean (sum / P) replaces the head's chunk-0 sums in place,
// which score_select_kernel then reads.
constexpr int kRowBlk = 256;
constexpr int kRowWaves = 16;
constexpr size_t kRowLds = 2 * (size_t)kRowBlk * 64 * sizeof(float);

__global__ void __launch_bounds__(64 * kRowWaves) score_rowsum_kernel(float* __restrict__ chunk_sums,
                                                                      int np, int P, int n_chunks) {
  extern __shared__ __align__(16) float rbuf[];  // [2][kRowBlk][64]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float* cs = chunk_sums + (int64_t)blockIdx.x * n_chunks * np;
  constexpr int per = kRowBlk / kRowWaves;  // chunks a wave loads per block
  float s = 0.0f;
  for (int c0 = 0, k = 0; c0 < n_chunks; c0 += kRowBlk, ++k) {
    float v[per];
#pragma unroll
    for (int j = 0; j < per; ++j) {  // chunk indices past the end are clamped (not added)
      const int c = min(c0 + wave + kRowWaves * j, n_chunks - 1);
      v[j] = lane < np ? cs[(int64_t)c * np + lane] : 0.0f;
    }
    __syncthreads();  // wave 0 has added the block that used this buffer
    float* buf = rbuf + (size_t)(k & 1) * kRowBlk * 64;
#pragma unroll
    for (int j = 0; j < per; ++j) buf[(wave + kRowWaves * j) * 64 + lane] = v[j];
    __syncthreads();
    if (wave == 0) {
      const int n = min(kRowBlk, n_chunks - c0);
#pragma unroll 8
      for (int c = 0; c < n; ++c) s = s + buf[c * 64 + lane];
    }
  }
  __syncthreads();  // every wave has read its chunk sums
  if (wave == 0 && lane < np) cs[lane] = s / (float)P;
}

__global__ void __launch_bounds__(1024) score_select_kernel(const float* __restrict__ chunk_sums,
                                                           float* __restrict__ sigma,
                                                           uint32_t* __restrict__ mask, int H_q,
                                                           int H_kv, int d, int P, int n_chunks,
                                                           int n_hi, int words, int presummed) {
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
    if (lane < np && presummed) {
      means[r][lane] = chunk_sums[((int64_t)(seq * H + head) * n_chunks) * np + lane];
    } else if (lane < np) {
      const float* cs = chunk_sums + ((int64_t)(seq * H + head) * n_chunks) * np + lane;
      // the adds stay in ascending chunk order; the loads go out kSelLoads at a time, and for
      // long prompts the next kSelLoads are in flight while the current ones are added (chunk
      // indices past the end are clamped to the last chunk: no load sits under a branch)
      auto ld = [&](float (&v)[kSelLoads], int c0) {
#pragma unroll
        for (int j = 0; j < kSelLoads; ++j) v[j] = cs[(int64_t)min(c0 + j, n_chunks - 1) * np];
      };
      float s = 0.0f;
      auto add = [&](const float (&v)[kSelLoads], int c0) {
#pragma unroll
        for (int j = 0; j < kSelLoads; ++j)
          if (c0 + j < n_chunks) s = s + v[j];
      };
      float va[kSelLoads];
      ld(va, 0);
      if (n_chunks <= kSelLoads) {
        add(va, 0);
      } else {
        float vb[kSelLoads];
        for (int c0 = 0;; c0 += 2 * kSelLoads) {
          ld(vb, c0 + kSelLoads);
          add(va, c0);
          if (c0 + kSelLoads >= n_chunks) break;
          ld(va, c0 + 2 * kSelLoads);
          add(vb, c0 + kSelLoads);
          if (c0 + 2 * kSelLoads >= n_chunks) break;
        }
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
                               const uint16_t* k, float* chunk_sums, int skip_Ns,
                               int skip_pages, hipStream_t stream) {
  const int n_chunks = (P + kChunk - 1) / kChunk;
  dim3 g1(B * (c.H_q + c.H_kv), n_chunks);
  switch (c.d) {
    case 32:
      hipLaunchKernelGGL(score_chunks_kernel<32>, g1, dim3(64), 0, stream, q, k, chunk_sums,
                         c.H_q, c.H_kv, c.pairing, P, n_chunks, skip_Ns, skip_pages);
      break;
    case 64:
      hipLaunchKernelGGL(score_chunks_kernel<64>, g1, dim3(64), 0, stream, q, k, chunk_sums,
                         c.H_q, c.H_kv, c.pairing, P, n_chunks, skip_Ns, skip_pages);
      break;
    case 128:
      hipLaunchKernelGGL(score_chunks_kernel<128>, g1, dim3(64), 0, stream, q, k, chunk_sums,
                         c.H_q, c.H_kv, c.pairing, P, n_chunks, skip_Ns, skip_pages);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_select(const pnmix_cfg& c, int B, int P, float* chunk_sums,
                               float* sigma, uint32_t* mask, hipStream_t stream) {
  const int n_chunks = (P + kChunk - 1) / kChunk;
  const int words = (c.d / 2 + 31) / 32;
  // long prompts: the chunk sums of every (sequence, head) are added by a workgroup of their
  // own first (rows in parallel; the means replace the chunk-0 sums), then one workgroup per
  // (sequence, KV head) ranks the pairs; short prompts: one kernel, four waves adding the rows
  int presummed = 0;
  if (n_chunks > kSelLoads && c.d / 2 <= 64) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&score_rowsum_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kRowLds);
    if (attr == hipSuccess) {
      hipLaunchKernelGGL(score_rowsum_kernel, dim3(B * (c.H_q + c.H_kv)), dim3(64 * kRowWaves),
                         kRowLds, stream, chunk_sums, c.d / 2, P, n_chunks);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      presummed = 1;
    }
  }
  const int rows = c.H_q / c.H_kv + 1;
  const int threads = !presummed && n_chunks > kSelLoads ? 64 * std::min(std::max(rows, 4), 16) : 256;
  hipLaunchKernelGGL(score_select_kernel, dim3(B * c.H_kv), dim3(threads), 0, stream, chunk_sums,
                     sigma, mask, c.H_q, c.H_kv, c.d, P, n_chunks, c.n_hi_pairs, words, presummed);
  return hipGetLastError();
}

hipError_t launch_score(const pnmix_cfg& c, int B, int P, const uint16_t* q, const uint16_t* k,
                        float* sigma, uint32_t* mask, void* ws, hipStream_t stream) {
  float* chunk_sums = static_cast<float*>(ws);
  const hipError_t e = launch_score_chunks(c, B, P, q, k, chunk_sums, 0, 0, stream);
  return e != hipSuccess ? e : launch_score_select(c, B, P, chunk_sums, sigma, mask, stream);
}

size_t score_workspace_bytes(const pnmix_cfg& c, int B, int P) {
  const size_t n_chunks = (size_t)(P + kChunk - 1) / kChunk;
  const size_t bytes = (size_t)B * (c.H_q + c.H_kv) * n_chunks * (c.d / 2) * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

}  // namespace pnmix
