// quant.hip -- key and value page quantization and bit packing on gfx950.
//
// PN-Mix paper (arXiv 2610.19605) sec. 2, Eq. 2: b-bit asymmetric min-max group quantization;
// keys grouped per channel along tokens, values per token along channels.  Reproduction notes
// ("PN-Mix: Key-Cache Precision Allocation from RoPE Channel-Pair Norms"), Core equations:
// Eq. 7 midpoint correction of 1-bit groups, zero scale plus the original offset for constant
// groups, H3/L1 packing.  Kernel-implementation appendix of the paper: LSB plane of every key
// channel at 8 tokens per byte, upper-2-bit plane of salient channels at 4 tokens per byte,
// values at 4 consecutive channels of one token per byte.
//
// One workgroup of 2d threads per page; thread (octet k, block b) holds tokens 8k..8k+7 x
// channels 8b..8b+7 of the N x d fp16 page in registers, read with one 16-byte load per token
// straight from HBM (each source byte read once, no LDS copy of the tile).
//   A. min / max of the thread's 8 x 8 values with packed fp16 min/max (exact), partials to LDS
//      (keys: per channel over the 8 tokens; values: per token over the 8 channels).
//   B. one thread per quantization group folds its partials, then takes the fp32 metadata
//      path of Eq. 2 / Eq. 7 (one IEEE divide, one IEEE reciprocal) and stores S, Z; the
//      group's (min, 1/s) go back through LDS.
//   C. per element q = rne(clamp((x - min) * (1/s), 0, L)): the clamp bounds are integers, so
//      clamping before rounding gives the same code as rounding first, and adding 2^23 to a
//      value in [0, L] rounds it to the nearest even integer and leaves it in the low
//      mantissa bits.  Key LSB bytes are packed in registers and stored as 8-byte runs; the
//      upper-bit plane (by salient rank) and the value bytes (formed in registers: a thread's 8
//      channels are two whole bytes of each of its tokens) are gathered in LDS and copied out
//      16 bytes a lane.
// Every float step is the reference arithmetic, so codes and fp16 metadata are bit-identical.
#include "common.h"
#include "kernels.h"
#include "quant_body.h"

namespace pnmix {
template <int D>
__global__ void __launch_bounds__(2 * D) quantize_k_kernel(const pnmix_page* __restrict__ jobs,
                                                          const uint32_t* __restrict__ mask,
                                                          int pairing, int n_hi, int G,
                                                          int words) {
  __shared__ __align__(16) uint8_t lds[KLds<D>::bytes];
  quantize_k_page<D>(jobs[blockIdx.x], mask, pairing, n_hi, G, words, lds);
}

template <int D>
__global__ void __launch_bounds__(2 * D) quantize_v_kernel(const pnmix_page* __restrict__ jobs,
                                                          int g_V) {
  __shared__ __align__(16) uint8_t lds[VLds<D>::bytes];
  quantize_v_page<D>(jobs[blockIdx.x], g_V, lds);
}

// Key and value pages in one launch: workgroup 2i takes key job i, workgroup 2i + 1 value job
// i, in one LDS allocation the size of the larger of the two, so the launch's last round is
// shared by both kinds of page.
template <int D>
__global__ void __launch_bounds__(2 * D) quantize_kv_kernel(const pnmix_page* __restrict__ kjobs,
                                                           const pnmix_page* __restrict__ vjobs,
                                                           const uint32_t* __restrict__ mask,
                                                           int pairing, int n_hi, int G,
                                                           int words, int g_V) {
  constexpr int bytes = KLds<D>::bytes > VLds<D>::bytes ? KLds<D>::bytes : VLds<D>::bytes;
  __shared__ __align__(16) uint8_t lds[bytes];
  const int i = blockIdx.x >> 1;
  if (blockIdx.x & 1)
    quantize_v_page<D>(vjobs[i], g_V, lds);
  else
    quantize_k_page<D>(kjobs[i], mask, pairing, n_hi, G, words, lds);
}

// ---------------------------------------------------------------------------------------------
// Every other bit width: (b_H, b_L) with 1 <= b_L <= b_H <= 4 and b_V in {1, 2, 4, 16} (the
// bit-width sweep of the PN-Mix paper's Table 14 / Figure 3).  Same arithmetic per group and
// element as above (exact min / max, group_meta, code_bits), so codes and metadata are again
// bit-identical to the reference; the layout generalises the appendix's planes: the low b_L
// bits of every key channel in a plane of width b_L, the upper b_H - b_L bits of the salient
// channels in a plane of that width (plane_field in common.h describes a plane), and 8 / b_V
// consecutive channels of one token per value byte.  One workgroup of 256 threads per page, the
// page staged in LDS; these kernels favour plainness over speed.


template <int D>
__global__ void __launch_bounds__(256) quantize_k_generic_kernel(
    const pnmix_page* __restrict__ jobs, const uint32_t* __restrict__ mask, int pairing, int n_hi,
    int G, int words, int bH, int bL) {
  __shared__ __align__(16) uint16_t xs[kN * D];
  __shared__ __align__(16) uint8_t q[kN * D];
  __shared__ float2 meta[(kN / 32) * D];
  __shared__ int rank_s[D];
  __shared__ int chan_s[D];
  const int tid = threadIdx.x;
  const pnmix_page job = jobs[blockIdx.x];
  const int n_sal = 2 * n_hi, wH = bH - bL, KG = kN / G;
  uint8_t* lo = job.dst;
  uint8_t* hi = lo + kN * D * bL / 8;
  uint16_t* S = reinterpret_cast<uint16_t*>(hi + kN * n_sal * wH / 8);
  uint16_t* Z = S + KG * D;
  stage_page<D>(xs, job.src, job.src_row_stride);
  const uint32_t* mrow = mask + job.mask_row * words;
  for (int c = tid; c < D; c += 256) {
    const int r = salient_rank(mrow, c, D, pairing, n_hi);
    rank_s[c] = r;
    if (r >= 0) chan_s[r] = c;
  }
  __syncthreads();
  for (int it = tid; it < KG * D; it += 256) {
    const int g = it / D, c = it % D;
    float mn = h2f(xs[(g * G) * D + c]), mx = mn;
    for (int t = g * G + 1; t < (g + 1) * G; ++t) {
      const float v = h2f(xs[t * D + c]);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    const int L = (1 << (rank_s[c] >= 0 ? bH : bL)) - 1;
    uint16_t s, z;
    meta[g * D + c] = group_meta(mn, mx, L, s, z);
    S[g * D + c] = s;
    Z[g * D + c] = z;
  }
  __syncthreads();
  for (int i = tid; i < kN * D; i += 256) {
    const int t = i / D, c = i % D;
    const float2 m = meta[(t / G) * D + c];
    const float L = (float)((1 << (rank_s[c] >= 0 ? bH : bL)) - 1);
    q[i] = (uint8_t)(code_bits(h2f(xs[i]), m.x, m.y, L) & 0xFFu);
  }
  __syncthreads();
  // low plane: unit (octet j, channel c) -> its b_L bytes
  for (int i = tid; i < (kN / 8) * D; i += 256) {
    const int j = i / D, c = i % D;
    uint32_t s = 0;
    for (int k = 0; k < 8; ++k) s |= ((uint32_t)q[(8 * j + k) * D + c] & ((1u << bL) - 1u)) << (bL * k);
    for (int b = 0; b < bL; ++b) lo[(j * bL + b) * D + c] = (uint8_t)(s >> (8 * b));
  }
  // high plane: unit (octet j, salient rank r) -> its b_H - b_L bytes
  if (wH > 0)
    for (int i = tid; i < (kN / 8) * n_sal; i += 256) {
      const int j = i / n_sal, r = i % n_sal, c = chan_s[r];
      uint32_t s = 0;
      for (int k = 0; k < 8; ++k) s |= ((uint32_t)q[(8 * j + k) * D + c] >> bL) << (wH * k);
      for (int b = 0; b < wH; ++b) hi[(j * wH + b) * n_sal + r] = (uint8_t)(s >> (8 * b));
    }
}

template <int D>
__global__ void __launch_bounds__(256) quantize_v_generic_kernel(const pnmix_page* __restrict__ jobs,
                                                                 int g_V, int bV) {
  __shared__ __align__(16) uint16_t xs[kN * D];
  __shared__ float2 meta[kN * 4];
  const int tid = threadIdx.x;
  const pnmix_page job = jobs[blockIdx.x];
  if (bV == 16) {  // values kept in fp16: the page is the rows [N][D]
    uint16_t* dst = reinterpret_cast<uint16_t*>(job.dst);
    for (int i = tid; i < kN * D; i += 256) dst[i] = job.src[(int64_t)(i / D) * job.src_row_stride + i % D];
    return;
  }
  const int ng = D / g_V, e = 8 / bV;
  uint8_t* codes = job.dst;
  uint16_t* S = reinterpret_cast<uint16_t*>(codes + kN * D * bV / 8);  // [ng][N]
  uint16_t* Z = S + kN * ng;
  stage_page<D>(xs, job.src, job.src_row_stride);
  __syncthreads();
  const int L = (1 << bV) - 1;
  for (int it = tid; it < kN * ng; it += 256) {
    const int t = it % kN, gi = it / kN;
    float mn = h2f(xs[t * D + gi * g_V]), mx = mn;
    for (int c = gi * g_V + 1; c < (gi + 1) * g_V; ++c) {
      const float v = h2f(xs[t * D + c]);
      mn = fminf(mn, v);
      mx = fmaxf(mx, v);
    }
    uint16_t s, z;
    meta[t * 4 + gi] = group_meta(mn, mx, L, s, z);
    S[gi * kN + t] = s;
    Z[gi * kN + t] = z;
  }
  __syncthreads();
  // byte [m][t]: channels e m .. e m + e - 1 of token t
  for (int i = tid; i < (D / e) * kN; i += 256) {
    const int m = i / kN, t = i % kN;
    uint32_t byte = 0;
    for (int u = 0; u < e; ++u) {
      const int c = e * m + u;
      const float2 mt = meta[t * 4 + c / g_V];
      byte |= (code_bits(h2f(xs[t * D + c]), mt.x, mt.y, (float)L) & 0xFFu) << (bV * u);
    }
    codes[i] = (uint8_t)byte;
  }
}

// Dequantized pages for analysis: x = S code + Z with the stored fp16 S and Z, one fma in fp32
// (the exact product and sum, rounded once).  One workgroup per page, out [N][D] f32.
template <int D>
__global__ void __launch_bounds__(256) dequant_k_kernel(const uint8_t* __restrict__ pages,
                                                        int64_t kpb, const uint32_t* __restrict__ mask,
                                                        int words, int pairing, int n_hi, int G,
                                                        int bH, int bL, float* __restrict__ out) {
  const uint8_t* pg = pages + (int64_t)blockIdx.x * kpb;
  const uint32_t* mrow = mask + (int64_t)blockIdx.x * words;
  const int n_sal = 2 * n_hi, wH = bH - bL;
  const uint8_t* hi = pg + kN * D * bL / 8;
  const uint8_t* Sp = hi + kN * n_sal * wH / 8;
  const uint8_t* Zp = Sp + 2 * (kN / G) * D;
  float* o = out + (int64_t)blockIdx.x * kN * D;
  for (int i = threadIdx.x; i < kN * D; i += 256) {
    const int t = i / D, c = i % D, g = t / G;
    uint32_t code = plane_field(pg, D, bL, c, t);
    const int r = salient_rank(mrow, c, D, pairing, n_hi);
    if (wH > 0 && r >= 0) code |= plane_field(hi, n_sal, wH, r, t) << bL;
    const float s = h2f(reinterpret_cast<const uint16_t*>(Sp)[g * D + c]);
    const float z = h2f(reinterpret_cast<const uint16_t*>(Zp)[g * D + c]);
    o[i] = __builtin_fmaf(s, (float)code, z);
  }
}

template <int D>
__global__ void __launch_bounds__(256) dequant_v_kernel(const uint8_t* __restrict__ pages,
                                                        int64_t vpb, int g_V, int bV,
                                                        float* __restrict__ out) {
  const uint8_t* pg = pages + (int64_t)blockIdx.x * vpb;
  float* o = out + (int64_t)blockIdx.x * kN * D;
  if (bV == 16) {
    for (int i = threadIdx.x; i < kN * D; i += 256) o[i] = h2f(reinterpret_cast<const uint16_t*>(pg)[i]);
    return;
  }
  const int e = 8 / bV, ng = D / g_V;
  const uint16_t* Sp = reinterpret_cast<const uint16_t*>(pg + kN * D * bV / 8);
  const uint16_t* Zp = Sp + ng * kN;
  for (int i = threadIdx.x; i < kN * D; i += 256) {
    const int t = i / D, c = i % D, g = c / g_V;
    const uint32_t code = (pg[(c / e) * kN + t] >> (bV * (c % e))) & ((1u << bV) - 1u);
    o[i] = __builtin_fmaf(h2f(Sp[g * kN + t]), (float)code, h2f(Zp[g * kN + t]));
  }
}

hipError_t launch_quantize_k(const pnmix_cfg& c, int n_pages, const pnmix_page* pages,
                             const uint32_t* mask, hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  const int words = (c.d / 2 + 31) / 32;
  const bool fast = c.b_H == 3 && c.b_L == 1;
#define PNMIX_QK(DD)                                                                             \
  if (fast)                                                                                      \
    hipLaunchKernelGGL(quantize_k_kernel<DD>, dim3(n_pages), dim3(2 * DD), 0, stream, pages, mask, \
                       c.pairing, c.n_hi_pairs, c.G, words);                                     \
  else                                                                                           \
    hipLaunchKernelGGL(quantize_k_generic_kernel<DD>, dim3(n_pages), dim3(256), 0, stream, pages, \
                       mask, c.pairing, c.n_hi_pairs, c.G, words, c.b_H, c.b_L);
  switch (c.d) {
    case 32: PNMIX_QK(32) break;
    case 64: PNMIX_QK(64) break;
    default: PNMIX_QK(128) break;
  }
#undef PNMIX_QK
  return hipGetLastError();
}

hipError_t launch_quantize_v(const pnmix_cfg& c, int n_pages, const pnmix_page* pages,
                             hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  const bool fast = c.b_V == 2;
#define PNMIX_QV(DD)                                                                             \
  if (fast)                                                                                      \
    hipLaunchKernelGGL(quantize_v_kernel<DD>, dim3(n_pages), dim3(2 * DD), 0, stream, pages, c.g_V); \
  else                                                                                           \
    hipLaunchKernelGGL(quantize_v_generic_kernel<DD>, dim3(n_pages), dim3(256), 0, stream, pages, \
                       c.g_V, c.b_V);
  switch (c.d) {
    case 32: PNMIX_QV(32) break;
    case 64: PNMIX_QV(64) break;
    default: PNMIX_QV(128) break;
  }
#undef PNMIX_QV
  return hipGetLastError();
}

hipError_t launch_quantize_kv(const pnmix_cfg& c, int n_pages, const pnmix_page* kjobs,
                              const pnmix_page* vjobs, const uint32_t* mask, hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  if (!(c.b_H == 3 && c.b_L == 1 && c.b_V == 2)) {  // the generic kernels: two launches
    const hipError_t e = launch_quantize_k(c, n_pages, kjobs, mask, stream);
    return e != hipSuccess ? e : launch_quantize_v(c, n_pages, vjobs, stream);
  }
  const int words = (c.d / 2 + 31) / 32;
  const dim3 grid(2 * n_pages);
  switch (c.d) {
    case 32:
      hipLaunchKernelGGL(quantize_kv_kernel<32>, grid, dim3(64), 0, stream, kjobs, vjobs, mask,
                         c.pairing, c.n_hi_pairs, c.G, words, c.g_V);
      break;
    case 64:
      hipLaunchKernelGGL(quantize_kv_kernel<64>, grid, dim3(128), 0, stream, kjobs, vjobs, mask,
                         c.pairing, c.n_hi_pairs, c.G, words, c.g_V);
      break;
    default:
      hipLaunchKernelGGL(quantize_kv_kernel<128>, grid, dim3(256), 0, stream, kjobs, vjobs, mask,
                         c.pairing, c.n_hi_pairs, c.G, words, c.g_V);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_dequant_k(const pnmix_cfg& c, int n_pages, const uint8_t* pages,
                            const uint32_t* mask, float* out, hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  const int words = (c.d / 2 + 31) / 32;
  const int64_t kpb = (int64_t)pnmix_k_page_bytes(&c);
#define PNMIX_DK(DD)                                                                             \
  hipLaunchKernelGGL(dequant_k_kernel<DD>, dim3(n_pages), dim3(256), 0, stream, pages, kpb, mask, \
                     words, c.pairing, c.n_hi_pairs, c.G, c.b_H, c.b_L, out);
  switch (c.d) {
    case 32: PNMIX_DK(32) break;
    case 64: PNMIX_DK(64) break;
    default: PNMIX_DK(128) break;
  }
#undef PNMIX_DK
  return hipGetLastError();
}

hipError_t launch_dequant_v(const pnmix_cfg& c, int n_pages, const uint8_t* pages, float* out,
                            hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  const int64_t vpb = (int64_t)pnmix_v_page_bytes(&c);
  switch (c.d) {
    case 32:
      hipLaunchKernelGGL(dequant_v_kernel<32>, dim3(n_pages), dim3(256), 0, stream, pages, vpb, c.g_V, c.b_V, out);
      break;
    case 64:
      hipLaunchKernelGGL(dequant_v_kernel<64>, dim3(n_pages), dim3(256), 0, stream, pages, vpb, c.g_V, c.b_V, out);
      break;
    default:
      hipLaunchKernelGGL(dequant_v_kernel<128>, dim3(n_pages), dim3(256), 0, stream, pages, vpb, c.g_V, c.b_V, out);
      break;
  }
  return hipGetLastError();
}

}  // namespace pnmix
