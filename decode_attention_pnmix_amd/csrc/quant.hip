// quant.hip -- key and value page quantization and bit packing on gfx950.
//
// PN-Mix paper (arXiv 2610.19605) sec. 2, Eq. 2: b-bit asymmetric min-max group quantization;
// keys grouped per channel along tokens, values per token along channels.  Reproduction notes
// ("PN-Mix: Key-Cache Precision Allocation from RoPE Channel-Pair Norms"), Core equations:
// Eq. 7 midpoint correction of 1-bit groups, zero scale plus original offset for constant
// groups, H3/L1 packing.  Kernel-implementation appendix of the paper: LSB plane of every key
// channel at 8 tokens per byte, upper-2-bit plane of salient channels at 4 tokens per byte,
// values at 4 channels per byte.
//
// One workgroup per page job.  The page's N x d fp16 tile is staged in LDS with 16-byte loads
// (each byte of the source read once), then each thread owns (channel, token group) items for
// keys or (token, channel group) items for values: exact min/max, one IEEE divide and one IEEE
// reciprocal per group, then per element sub, mul, round-half-even, clamp -- the reference
// arithmetic, so codes and fp16 metadata are bit-identical to the oracle.
#include "common.h"
#include "kernels.h"

namespace pnmix {

constexpr int kQuantThreads = 256;
constexpr int kMaxD = 128;
constexpr int kN = 128;

// Copy one N x d fp16 page (row stride in elements) into LDS, 16 bytes per access when the
// source is 16-byte aligned with a stride that keeps rows aligned, else 2 bytes per access.
__device__ __forceinline__ void stage_page(uint16_t* tile, const uint16_t* src, int64_t stride,
                                           int d) {
  const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15) == 0) && ((stride & 7) == 0);
  if (vec) {
    const int per_row = d / 8;
    for (int i = threadIdx.x; i < kN * per_row; i += blockDim.x) {
      const int t = i / per_row, c8 = i % per_row;
      const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)t * stride + c8 * 8);
      *reinterpret_cast<uint4*>(tile + t * d + c8 * 8) = v;
    }
  } else {
    for (int i = threadIdx.x; i < kN * d; i += blockDim.x) {
      const int t = i / d, c = i % d;
      tile[t * d + c] = src[(int64_t)t * stride + c];
    }
  }
}

struct GroupQ {
  float mn, inv;
  int L;
  bool constant;
  uint16_t S, Z;
};

// Eq. 2 / Eq. 7 metadata of one group from its exact min and max.
__device__ __forceinline__ GroupQ group_params(float mn, float mx, int bits) {
  GroupQ g;
  g.mn = canon(mn);
  mx = canon(mx);
  g.L = (1 << bits) - 1;
  g.constant = (mx == g.mn);
  if (g.constant) {
    g.inv = 0.0f;
    g.S = 0;
    g.Z = f2h(g.mn);
    return g;
  }
  const float s = (mx - g.mn) / (float)g.L;
  g.inv = 1.0f / s;
  if (g.L == 1) {
    const float s7 = (mx - g.mn) * 0.5f;
    const float t3 = 3.0f * g.mn;
    const float z7 = (t3 + mx) * 0.25f;
    g.S = f2h(s7);
    g.Z = f2h(z7);
  } else {
    g.S = f2h(s);
    g.Z = f2h(g.mn);
  }
  return g;
}

__device__ __forceinline__ uint32_t group_code(const GroupQ& g, float x) {
  if (g.constant) return 0u;
  float r = rintf((x - g.mn) * g.inv);
  r = fminf(fmaxf(r, 0.0f), (float)g.L);
  return (uint32_t)(int)r;
}

__global__ void __launch_bounds__(kQuantThreads) quantize_k_kernel(const pnmix_page* __restrict__ jobs,
                                                                   const uint32_t* __restrict__ mask,
                                                                   int d, int pairing, int n_hi,
                                                                   int G, int words) {
  __shared__ __align__(16) uint16_t tile[kN * kMaxD];
  const pnmix_page job = jobs[blockIdx.x];
  stage_page(tile, job.src, job.src_row_stride, d);
  __syncthreads();
  const uint32_t* mrow = mask + job.mask_row * words;
  const int n_sal = 2 * n_hi;
  uint8_t* lo = job.dst;
  uint8_t* hi = lo + kN * d / 8;
  uint16_t* S = reinterpret_cast<uint16_t*>(hi + kN * n_sal / 4);
  uint16_t* Z = S + (kN / G) * d;
  const int items = d * (kN / G);
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int c = it % d, g = it / d;
    const int rank = salient_rank(mrow, c, d, pairing, n_hi);
    const uint16_t* col = tile + g * G * d + c;
    float mn = h2f(col[0]), mx = mn;
    for (int t = 1; t < G; ++t) {
      const float v = h2f(col[t * d]);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    const GroupQ q = group_params(mn, mx, rank >= 0 ? 3 : 1);
    for (int j = 0; j < G / 8; ++j) {
      uint32_t lob = 0u, hib0 = 0u, hib1 = 0u;
      for (int k = 0; k < 8; ++k) {
        const uint32_t code = group_code(q, h2f(col[(8 * j + k) * d]));
        lob |= (code & 1u) << k;
        if (k < 4)
          hib0 |= (code >> 1) << (2 * k);
        else
          hib1 |= (code >> 1) << (2 * (k - 4));
      }
      lo[(g * G / 8 + j) * d + c] = (uint8_t)lob;
      if (rank >= 0) {
        hi[(g * G / 4 + 2 * j) * n_sal + rank] = (uint8_t)hib0;
        hi[(g * G / 4 + 2 * j + 1) * n_sal + rank] = (uint8_t)hib1;
      }
    }
    S[g * d + c] = q.S;
    Z[g * d + c] = q.Z;
  }
}

__global__ void __launch_bounds__(kQuantThreads) quantize_v_kernel(const pnmix_page* __restrict__ jobs,
                                                                   int d, int g_V) {
  __shared__ __align__(16) uint16_t tile[kN * kMaxD];
  const pnmix_page job = jobs[blockIdx.x];
  stage_page(tile, job.src, job.src_row_stride, d);
  __syncthreads();
  const int ng = d / g_V;
  uint8_t* codes = job.dst;
  uint16_t* S = reinterpret_cast<uint16_t*>(codes + kN * d / 4);  // [ng][N]
  uint16_t* Z = S + kN * ng;                                        // [ng][N]
  for (int it = threadIdx.x; it < kN * ng; it += blockDim.x) {
    const int gi = it % ng, t = it / ng;
    const uint16_t* row = tile + t * d + gi * g_V;
    float mn = h2f(row[0]), mx = mn;
    for (int c = 1; c < g_V; ++c) {
      const float v = h2f(row[c]);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    const GroupQ q = group_params(mn, mx, 2);
    for (int m = 0; m < g_V / 4; ++m) {
      uint32_t byte = 0u;
      for (int u = 0; u < 4; ++u) byte |= group_code(q, h2f(row[4 * m + u])) << (2 * u);
      const int mcol = gi * g_V / 4 + m;
      codes[((t / 8) * (d / 4) + mcol) * 8 + (t % 8)] = (uint8_t)byte;
    }
    S[gi * kN + t] = q.S;
    Z[gi * kN + t] = q.Z;
  }
}

hipError_t launch_quantize_k(const pnmix_cfg& c, int n_pages, const pnmix_page* pages,
                             const uint32_t* mask, hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  const int words = (c.d / 2 + 31) / 32;
  hipLaunchKernelGGL(quantize_k_kernel, dim3(n_pages), dim3(kQuantThreads), 0, stream, pages,
                     mask, c.d, c.pairing, c.n_hi_pairs, c.G, words);
  return hipGetLastError();
}

hipError_t launch_quantize_v(const pnmix_cfg& c, int n_pages, const pnmix_page* pages,
                             hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_v_kernel, dim3(n_pages), dim3(kQuantThreads), 0, stream, pages,
                     c.d, c.g_V);
  return hipGetLastError();
}

}  // namespace pnmix
