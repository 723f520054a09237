// prefill.hip -- prefill scoring and the prompt's page quantization with one read of the keys.
//
// PN-Mix paper (arXiv 2610.19605) sec. 5 and the Korean summary page ("무엇과 다른가"): the
// salient RoPE pairs are chosen once from the prefill tokens (Eq. 6 of the reproduction notes
// "PN-Mix: Key-Cache Precision Allocation from RoPE Channel-Pair Norms") and every page of the
// key cache is quantized with that mask, the prompt's own full pages included.  Scoring and then
// quantizing reads the prompt's keys twice.  Here they are read once.  The mask depends on
// every prompt token, so a workgroup holding a page cannot know it yet: it forms both encodings
// a key channel can take (the 3-bit codes of a salient channel, the 1-bit Eq. 7 codes of the
// others) with their metadata, and a last kernel assembles the page once the mask exists.
// Launches:
//   1. score.hip's chunk kernel: chunk sums of the query heads, and of the key chunks that do not
//      lie wholly inside one full page (those among the sinks, across a page boundary, or after
//      the last full page);
//   2. one workgroup per (sequence, KV head, prompt page): the page's 128 token rows go to LDS
//      once; the key chunk sums of the chunks lying inside the page (the score kernel's
//      arithmetic and order: per token sqrt(x x + y y) correctly rounded, ascending tokens from
//      +0); per (token group, channel) the exact min and max and the metadata of both bit widths
//      (quant_body.h's group_meta); then, per 8 tokens and 4 channels, both code sets packed
//      (the 1-bit LSB bytes, the 3-bit codes' LSB bytes and their two upper-bit bytes), staged
//      in LDS and written with 16-byte stores;
//   3. the value pages (the mask plays no part in them): quant_body.h's value page body;
//   4. score.hip's select kernel: sigma and the mask;
//   5. one workgroup per page: the LSB plane takes each channel's 3-bit or 1-bit byte by the
//      mask, the upper-bit plane gathers the salient channels' bytes in rank order, S and Z
//      follow the same choice.  Codes and metadata are those of pnmix_quantize_k_page bit for
//      bit (same min, max, metadata and code arithmetic per element).
#include "common.h"
#include "kernels.h"
#include "quant_body.h"

namespace pnmix {

constexpr int kChunkTokens = 64;  // score chunk length (score.hip)

// Candidate encodings of one key page in the workspace: LSB plane of the 1-bit codes [N/8][d],
// LSB plane of the 3-bit codes [N/8][d], upper-2-bit plane of the 3-bit codes for every channel
// [N/4][d], then S1, Z1, S3, Z3 [N/G][d] fp16.
__host__ __device__ constexpr int cand_bytes(int d, int KG) { return kN * d / 2 + 8 * KG * d; }

struct PrefillArgs {
  const uint16_t* k;    // [B][H_kv][P][d]
  const uint16_t* v;
  uint8_t* k_pages;     // [B][max_pages][H_kv][kpb]
  uint8_t* v_pages;
  const uint32_t* mask; // [B][H_kv][words] (finalize)
  float* chunk_sums;    // score layout [B * (H_q + H_kv)][n_chunks][d/2]
  uint8_t* cand;        // [B * H_kv * n_full][cand_bytes]
  int H_q, H_kv, P, N_s, n_full, n_chunks, max_pages, pairing, n_hi, G, g_V, words;
  int64_t kpb, vpb;
};

template <int D>
__global__ void __launch_bounds__(2 * D) prefill_k_pages_kernel(PrefillArgs a) {
  constexpr int NP = D / 2;
  constexpr int QD = D / 4;                         // channel quads
  constexpr int kUnits = (kN / 8) * QD / (2 * D);   // (octet, quad) units per thread: 2
  __shared__ __align__(16) uint16_t tile[kN * D];   // the page's rows, then the staged codes
  __shared__ __align__(16) float4 meta[(kN / 32) * D];  // (mn, 1/s of L = 1, 1/s of L = 7)
  const int tid = threadIdx.x;
  const int p = blockIdx.x % a.n_full;
  const int64_t bh = blockIdx.x / a.n_full;
  const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
  const int KG = kN / a.G;
  const int tok0 = a.N_s + kN * p;
  const uint16_t* src = a.k + (bh * a.P + tok0) * D;
  // the page's rows -> LDS (16-byte pieces; rows of d fp16 are 16-byte multiples), every load
  // issued before the first store
  if ((reinterpret_cast<uintptr_t>(src) & 15) == 0) {
    constexpr int kLoads = kN * D / 8 / (2 * D);
    uint4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) v[j] = reinterpret_cast<const uint4*>(src)[tid + 2 * D * j];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) reinterpret_cast<uint4*>(tile)[tid + 2 * D * j] = v[j];
  } else {
    for (int i = tid; i < kN * D; i += 2 * D) tile[i] = src[i];
  }
  __syncthreads();

  // key chunk sums of the chunks lying wholly inside this page: thread (pair i, chunk cf + j)
  {
    const int i = tid % NP, j = tid / NP;
    const int cf = (tok0 + kChunkTokens - 1) / kChunkTokens;
    const int c = cf + j;
    if (kChunkTokens * (c + 1) <= tok0 + kN) {
      const int ch0 = a.pairing == PNMIX_PAIRS_ADJACENT ? 2 * i : i;
      const int ch1 = a.pairing == PNMIX_PAIRS_ADJACENT ? 2 * i + 1 : i + NP;
      const int r0 = kChunkTokens * c - tok0;
      float s = 0.0f;
#pragma unroll 8
      for (int t = 0; t < kChunkTokens; ++t)
        s = s + pair_norm(tile[(r0 + t) * D + ch0], tile[(r0 + t) * D + ch1]);
      const int64_t head = (int64_t)b * (a.H_q + a.H_kv) + a.H_q + h;
      a.chunk_sums[(head * a.n_chunks + c) * NP + i] = s;
    }
  }

  // metadata of both bit widths per (token group, channel)
  uint8_t* cd = a.cand + ((bh * a.n_full) + p) * (int64_t)cand_bytes(D, KG);
  uint16_t* S1 = reinterpret_cast<uint16_t*>(cd + kN * D / 2);
  uint16_t* Z1 = S1 + KG * D;
  uint16_t* S3 = Z1 + KG * D;
  uint16_t* Z3 = S3 + KG * D;
  for (int it = tid; it < KG * D; it += 2 * D) {
    const int g = it / D, c = it % D;
    float mn = h2f(tile[(g * a.G) * D + c]), mx = mn;
    for (int t = g * a.G + 1; t < (g + 1) * a.G; ++t) {
      const float x = h2f(tile[t * D + c]);
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    uint16_t s1, z1, s3, z3;
    const float2 m1 = group_meta(mn, mx, 1, s1, z1);
    const float2 m3 = group_meta(mn, mx, 7, s3, z3);
    meta[it] = make_float4(m1.x, m1.y, m3.y, 0.0f);
    S1[it] = s1;
    Z1[it] = z1;
    S3[it] = s3;
    Z3[it] = z3;
  }
  __syncthreads();

  // both code sets, packed in registers: unit (octet j, channel quad m) = tokens 8j..8j+7 of
  // channels 4m..4m+3; byte e of each word belongs to channel 4m + e
  uint32_t w_l1[kUnits], w_l3[kUnits], w_u0[kUnits], w_u1[kUnits];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const int it = tid + 2 * D * u;
    const int j = it / QD, m = it % QD;
    float4 mt[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) mt[e] = meta[((8 * j) / a.G) * D + 4 * m + e];
    uint32_t l1 = 0, l3 = 0, u0 = 0, u1 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint2 x4 = *reinterpret_cast<const uint2*>(tile + (8 * j + k) * D + 4 * m);
      const uint16_t xs[4] = {(uint16_t)(x4.x & 0xFFFFu), (uint16_t)(x4.x >> 16),
                              (uint16_t)(x4.y & 0xFFFFu), (uint16_t)(x4.y >> 16)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = h2f(xs[e]);
        const uint32_t q1 = code_bits(x, mt[e].x, mt[e].y, 1.0f) & 0xFFu;
        const uint32_t q3 = code_bits(x, mt[e].x, mt[e].z, 7.0f) & 0xFFu;
        l1 |= (q1 & 1u) << (8 * e + k);
        l3 |= (q3 & 1u) << (8 * e + k);
        if (k < 4)
          u0 |= (q3 >> 1) << (8 * e + 2 * k);
        else
          u1 |= (q3 >> 1) << (8 * e + 2 * (k - 4));
      }
    }
    w_l1[u] = l1;
    w_l3[u] = l3;
    w_u0[u] = u0;
    w_u1[u] = u1;
  }
  __syncthreads();  // the rows are read: the tile takes the packed planes
  uint8_t* st = reinterpret_cast<uint8_t*>(tile);
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const int it = tid + 2 * D * u;
    const int j = it / QD, m = it % QD;
    *reinterpret_cast<uint32_t*>(st + j * D + 4 * m) = w_l1[u];
    *reinterpret_cast<uint32_t*>(st + kN * D / 8 + j * D + 4 * m) = w_l3[u];
    *reinterpret_cast<uint32_t*>(st + kN * D / 4 + (2 * j) * D + 4 * m) = w_u0[u];
    *reinterpret_cast<uint32_t*>(st + kN * D / 4 + (2 * j + 1) * D + 4 * m) = w_u1[u];
  }
  __syncthreads();
  // LSB planes [N/8][D] (1-bit, then 3-bit) and the upper-bit plane [N/4][D]: N D / 2 bytes
  for (int i = tid; i < kN * D / 32; i += 2 * D)
    reinterpret_cast<uint4*>(cd)[i] = reinterpret_cast<const uint4*>(st)[i];
}

template <int D>
__global__ void __launch_bounds__(2 * D) prefill_v_pages_kernel(PrefillArgs a) {
  __shared__ __align__(16) uint8_t lds[VLds<D>::bytes];
  const int p = blockIdx.x % a.n_full;
  const int64_t bh = blockIdx.x / a.n_full;
  const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
  pnmix_page job;
  job.src = a.v + (bh * a.P + a.N_s + kN * p) * D;
  job.src_row_stride = D;
  job.dst = a.v_pages + (((int64_t)b * a.max_pages + p) * a.H_kv + h) * a.vpb;
  job.mask_row = 0;
  quantize_v_page<D>(job, a.g_V, lds);
}

template <int D>
__global__ void __launch_bounds__(256) prefill_k_finalize_kernel(PrefillArgs a) {
  __shared__ int rank_s[D];
  __shared__ int chan_s[D];
  // the page's candidates (both LSB planes and the upper-bit plane of every channel, N D / 2
  // bytes, with 16-byte loads), then the final page assembled in LDS and stored with 16-byte
  // stores (its planes and metadata are 16-byte multiples for every supported shape)
  __shared__ __align__(16) uint8_t cin[kN * D / 2];
  __shared__ __align__(16) uint8_t pout[kN * D / 8 + kN * D / 4];
  const int tid = threadIdx.x;
  const int p = blockIdx.x % a.n_full;
  const int64_t bh = blockIdx.x / a.n_full;
  const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
  const int KG = kN / a.G, n_sal = 2 * a.n_hi;
  const uint32_t* mrow = a.mask + bh * a.words;
  const uint8_t* cd = a.cand + ((bh * a.n_full) + p) * (int64_t)cand_bytes(D, KG);
  for (int i = tid; i < kN * D / 32; i += 256)
    reinterpret_cast<uint4*>(cin)[i] = reinterpret_cast<const uint4*>(cd)[i];
  for (int c = tid; c < D; c += 256) chan_s[c] = 0;  // every rank names a channel
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    const int r = salient_rank(mrow, c, D, a.pairing, a.n_hi);
    rank_s[c] = r;
    if (r >= 0) chan_s[r] = c;
  }
  __syncthreads();
  const uint8_t* lsb1 = cin;
  const uint8_t* lsb3 = cin + kN * D / 8;
  const uint8_t* hi3 = cin + kN * D / 4;
  const uint16_t* S1 = reinterpret_cast<const uint16_t*>(cd + kN * D / 2);
  const uint16_t* Z1 = S1 + KG * D;
  const uint16_t* S3 = Z1 + KG * D;
  const uint16_t* Z3 = S3 + KG * D;
  uint8_t* dst = a.k_pages + (((int64_t)b * a.max_pages + p) * a.H_kv + h) * a.kpb;
  const int lo_bytes = kN * D / 8, hi_bytes = kN * n_sal / 4;
  for (int i = tid; i < lo_bytes; i += 256) pout[i] = rank_s[i % D] >= 0 ? lsb3[i] : lsb1[i];
  for (int i = tid; i < hi_bytes; i += 256) {
    const int j = i / n_sal, r = i % n_sal;
    pout[lo_bytes + i] = hi3[j * D + chan_s[r]];
  }
  uint16_t* S = reinterpret_cast<uint16_t*>(dst + lo_bytes + hi_bytes);
  uint16_t* Z = S + KG * D;
  for (int i = tid; i < KG * D; i += 256) {
    const bool sal = rank_s[i % D] >= 0;
    S[i] = sal ? S3[i] : S1[i];
    Z[i] = sal ? Z3[i] : Z1[i];
  }
  __syncthreads();
  // lo and hi planes: (N D / 8 + N n_sal / 4) bytes, a multiple of 16 (n_sal is even, N = 128)
  for (int i = tid; i < (lo_bytes + hi_bytes) / 16; i += 256)
    reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(pout)[i];
}

static int prefill_pages(const pnmix_cfg& c, int P) { return P > c.N_s ? (P - c.N_s) / kN : 0; }

size_t prefill_workspace_bytes(const pnmix_cfg& c, int B, int P) {
  const size_t cand = (size_t)B * c.H_kv * prefill_pages(c, P) * cand_bytes(c.d, kN / c.G);
  return score_workspace_bytes(c, B, P) + ((cand + 255) & ~(size_t)255);
}

hipError_t launch_prefill_fused(const pnmix_cfg& c, int B, int P, const uint16_t* q,
                                const uint16_t* k, const uint16_t* v, float* sigma,
                                uint32_t* mask, uint8_t* k_pages, uint8_t* v_pages,
                                int max_pages, void* ws, hipStream_t stream) {
  const int n_full = prefill_pages(c, P);
  PrefillArgs a;
  a.k = k;
  a.v = v;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.mask = mask;
  a.chunk_sums = static_cast<float*>(ws);
  a.cand = static_cast<uint8_t*>(ws) + score_workspace_bytes(c, B, P);
  a.H_q = c.H_q;
  a.H_kv = c.H_kv;
  a.P = P;
  a.N_s = c.N_s;
  a.n_full = n_full;
  a.n_chunks = (P + kChunkTokens - 1) / kChunkTokens;
  a.max_pages = max_pages;
  a.pairing = c.pairing;
  a.n_hi = c.n_hi_pairs;
  a.G = c.G;
  a.g_V = c.g_V;
  a.words = (c.d / 2 + 31) / 32;
  a.kpb = (int64_t)pnmix_k_page_bytes(&c);
  a.vpb = (int64_t)pnmix_v_page_bytes(&c);
  // key chunks lying wholly inside a full page come from the page workgroups
  hipError_t e = launch_score_chunks(c, B, P, q, k, a.chunk_sums, c.N_s, n_full, stream);
  if (e != hipSuccess) return e;
  const dim3 pages((unsigned)B * c.H_kv * n_full);
  if (n_full > 0) {
    switch (c.d) {
      case 32:
        hipLaunchKernelGGL(prefill_k_pages_kernel<32>, pages, dim3(64), 0, stream, a);
        hipLaunchKernelGGL(prefill_v_pages_kernel<32>, pages, dim3(64), 0, stream, a);
        break;
      case 64:
        hipLaunchKernelGGL(prefill_k_pages_kernel<64>, pages, dim3(128), 0, stream, a);
        hipLaunchKernelGGL(prefill_v_pages_kernel<64>, pages, dim3(128), 0, stream, a);
        break;
      default:
        hipLaunchKernelGGL(prefill_k_pages_kernel<128>, pages, dim3(256), 0, stream, a);
        hipLaunchKernelGGL(prefill_v_pages_kernel<128>, pages, dim3(256), 0, stream, a);
        break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  e = launch_score_select(c, B, P, a.chunk_sums, sigma, mask, stream);
  if (e != hipSuccess || n_full == 0) return e;
  switch (c.d) {
    case 32: hipLaunchKernelGGL(prefill_k_finalize_kernel<32>, pages, dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(prefill_k_finalize_kernel<64>, pages, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(prefill_k_finalize_kernel<128>, pages, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace pnmix
