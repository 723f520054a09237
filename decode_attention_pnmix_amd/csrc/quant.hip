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
// bit-width sweep of the PN-Mix paper's Table 14 / Figure 3).  The same register tiles, steps
// and per-element arithmetic as above (exact min / max, group_meta, code_bits_h), so codes and
// metadata are again bit-identical to the reference; the layout generalises the appendix's
// planes: the low b_L bits of every key channel in a plane of width b_L, the upper b_H - b_L bits
// of the salient channels in a plane of that width (a plane stores the w-bit fields of tokens
// 8j .. 8j + 7 of a column as one 8w-bit little-endian stream in w bytes; plane_field in common.h),
// and 8 / b_V consecutive channels of one token per value byte.

// byte i of each of four words -> one word (w0's in byte 0)
__device__ __forceinline__ uint32_t gather_bi(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                              int i) {
  const uint32_t sel = 0x0c0c0000u | (uint32_t)(4 + i) << 8 | (uint32_t)i;  // [w0.bi, w1.bi, 0, 0]
  return perm(perm(w3, w2, sel), perm(w1, w0, sel), 0x05040100u);
}

// LDS of one key page, any widths: (min, max) per octet and channel, (min, 1/s) per group and
// channel, the upper plane (at most 3 bits: N / 8 octets x 3 bytes x d ranks), salient ranks.
template <int D>
struct KWLds {
  static constexpr int part = 0;
  static constexpr int meta = part + kOctets * D * 4;
  static constexpr int hi = meta + (kN / 32) * D * 8;
  static constexpr int rank = hi + kOctets * 3 * D;
  static constexpr int bytes = rank + D;
};

template <int D>
__device__ __forceinline__ void quantize_k_page_w(const pnmix_page& job,
                                                  const uint32_t* __restrict__ mask, int pairing,
                                                  int n_hi, int G, int words, int bH, int bL,
                                                  uint8_t* lds) {
  constexpr int NB = D / 8;
  uint32_t* part = reinterpret_cast<uint32_t*>(lds + KWLds<D>::part);
  float2* meta = reinterpret_cast<float2*>(lds + KWLds<D>::meta);
  uint8_t* hi_s = lds + KWLds<D>::hi;
  int8_t* rank_s = reinterpret_cast<int8_t*>(lds + KWLds<D>::rank);
  const int tid = threadIdx.x, b = tid % NB, k = tid / NB;
  const int n_sal = 2 * n_hi, wH = bH - bL;
  uint8_t* lo = job.dst;
  uint8_t* hi = lo + kN * D * bL / 8;
  uint16_t* S = reinterpret_cast<uint16_t*>(hi + kN * n_sal * wH / 8);
  uint16_t* Z = S + (kN / G) * D;

  uint4 x[8];
  load_block(x, job.src, job.src_row_stride, k, b);

  // A: per channel min / max over the 8 tokens
  {
    uint32_t pm[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t mn = word(x[0], m), mx = mn;
#pragma unroll
      for (int j = 1; j < 8; ++j) {
        mn = pk_min(mn, word(x[j], m));
        mx = pk_max(mx, word(x[j], m));
      }
      pm[2 * m] = perm(mx, mn, 0x05040100u);
      pm[2 * m + 1] = perm(mx, mn, 0x07060302u);
    }
    uint4* dst = reinterpret_cast<uint4*>(part + k * D + 8 * b);
    dst[0] = make_uint4(pm[0], pm[1], pm[2], pm[3]);
    dst[1] = make_uint4(pm[4], pm[5], pm[6], pm[7]);
  }
  const uint32_t* mrow = mask + job.mask_row * words;
  if (tid < D) rank_s[tid] = (int8_t)salient_rank(mrow, tid, D, pairing, n_hi);
  __syncthreads();

  // B: one thread per (token group, channel)
  const int og = G / 8;
  for (int it = tid; it < (kN / G) * D; it += 2 * D) {
    const int g = it / D, c = it % D;
    float mn = lo_f(part[g * og * D + c]), mx = hi_f(part[g * og * D + c]);
    for (int o = 1; o < og; ++o) {
      const uint32_t v = part[(g * og + o) * D + c];
      mn = fminf(mn, lo_f(v));
      mx = fmaxf(mx, hi_f(v));
    }
    const int L = (1 << (rank_s[c] >= 0 ? bH : bL)) - 1;
    uint16_t s, z;
    meta[g * D + c] = group_meta(mn, mx, L, s, z);
    S[g * D + c] = s;
    Z[g * D + c] = z;
  }
  __syncthreads();

  // C: codes of the thread's 8 channels x 8 tokens, as the bit streams of the two planes
  const int g = k / og;
  const uint32_t mL = (1u << bL) - 1u;
  uint32_t lob[8];  // channel s: the 8 b_L-bit fields of the octet, token j at bit b_L j
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float2 mt = meta[g * D + 8 * b + s];
    const int rk = rank_s[8 * b + s];
    const float L = (float)((1 << (rk >= 0 ? bH : bL)) - 1);
    uint32_t sl = 0, sh = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t q = code_bits_h(word(x[j], s >> 1), (s & 1) != 0, -mt.x, mt.y, L) & 15u;
      sl |= (q & mL) << (bL * j);
      sh |= (q >> bL) << (wH * j);
    }
    lob[s] = sl;
    if (wH > 0 && rk >= 0)
      for (int i = 0; i < wH; ++i) hi_s[(k * wH + i) * n_sal + rk] = (uint8_t)(sh >> (8 * i));
  }
  for (int i = 0; i < bL; ++i) {
    const uint32_t w0 = gather_bi(lob[0], lob[1], lob[2], lob[3], i);
    const uint32_t w1 = gather_bi(lob[4], lob[5], lob[6], lob[7], i);
    *reinterpret_cast<uint2*>(lo + (k * bL + i) * D + 8 * b) = make_uint2(w0, w1);
  }
  __syncthreads();
  if (wH > 0) {
    const int hi_chunks = kOctets * wH * n_sal / 16;  // 16 w_H n_sal bytes
    for (int i = tid; i < hi_chunks; i += 2 * D)
      reinterpret_cast<uint4*>(hi)[i] = reinterpret_cast<const uint4*>(hi_s)[i];
  }
}

// LDS of one value page, any widths: (min, max) per token and 8-channel block, (min, 1/s) per
// token and group (<= 4)
template <int D>
struct VWLds {
  static constexpr int part = 0;
  static constexpr int meta = part + kN * (D / 8) * 4;
  static constexpr int bytes = meta + kN * 4 * 8;
};

template <int D, int BV>
__device__ __forceinline__ void quantize_v_page_w(const pnmix_page& job, int g_V, uint8_t* lds) {
  constexpr int NB = D / 8;
  const int tid = threadIdx.x, b = tid % NB, k = tid / NB;
  uint4 x[8];
  load_block(x, job.src, job.src_row_stride, k, b);
  if constexpr (BV == 16) {  // values kept in fp16: the page is the rows [N][D]
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<uint4*>(job.dst + 2 * ((8 * k + j) * D + 8 * b)) = x[j];
    return;
  }
  constexpr int bV = BV == 16 ? 8 : BV, e = 8 / bV;  // code bits; codes per byte
  uint32_t* part = reinterpret_cast<uint32_t*>(lds + VWLds<D>::part);
  float2* meta = reinterpret_cast<float2*>(lds + VWLds<D>::meta);
  const int ng = D / g_V;
  uint8_t* codes = job.dst;
  uint16_t* S = reinterpret_cast<uint16_t*>(codes + kN * D * bV / 8);  // [ng][N]
  uint16_t* Z = S + kN * ng;

  // A: per token min / max over the thread's 8 channels
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t mn2 = pk_min(pk_min(x[j].x, x[j].y), pk_min(x[j].z, x[j].w));
    const uint32_t mx2 = pk_max(pk_max(x[j].x, x[j].y), pk_max(x[j].z, x[j].w));
    const _Float16 mn = __builtin_elementwise_min(as_h2(mn2).x, as_h2(mn2).y);
    const _Float16 mx = __builtin_elementwise_max(as_h2(mx2).x, as_h2(mx2).y);
    part[(8 * k + j) * NB + b] = (uint32_t)__builtin_bit_cast(uint16_t, mn) |
                                 ((uint32_t)__builtin_bit_cast(uint16_t, mx) << 16);
  }
  __syncthreads();

  // B: one thread per (token, channel group)
  const int bg = g_V / 8;
  const int L = (1 << bV) - 1;
  for (int it = tid; it < kN * ng; it += 2 * D) {
    const int t = it % kN, gi = it / kN;
    const uint32_t* pr = part + t * NB + gi * bg;
    float mn = lo_f(pr[0]), mx = hi_f(pr[0]);
    for (int o = 1; o < bg; ++o) {
      mn = fminf(mn, lo_f(pr[o]));
      mx = fmaxf(mx, hi_f(pr[o]));
    }
    uint16_t s, z;
    meta[t * 4 + gi] = group_meta(mn, mx, L, s, z);
    S[gi * kN + t] = s;
    Z[gi * kN + t] = z;
  }
  __syncthreads();

  // C: codes of the thread's 8 tokens x 8 channels: channels 8b .. 8b + 7 are the b_V byte
  // columns 8b / e .. 8b / e + b_V - 1 of each token.  A code is the low byte of its float
  // 2^23 + q, so the sum of the codes shifted to their fields has the byte in its low 8 bits.
  const int gi = b / bg;
  const float Lf = (float)L;
  static_assert(BV == 1 || BV == 2 || BV == 4 || BV == 16, "value width");
  uint32_t by[bV][8];  // [byte column 8b / e + h][token]
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float2 mt = meta[(8 * k + t) * 4 + gi];
    uint32_t cu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) cu[i] = code_bits_h(word(x[t], i >> 1), (i & 1) != 0, -mt.x, mt.y, Lf);
#pragma unroll
    for (int h = 0; h < bV; ++h) {
      uint32_t v = 0;
#pragma unroll
      for (int u = 0; u < e; ++u) v += cu[e * h + u] << (bV * u);
      by[h][t] = v;
    }
  }
#pragma unroll
  for (int h = 0; h < bV; ++h)
    *reinterpret_cast<uint2*>(codes + (8 * b / e + h) * kN + 8 * k) =
        make_uint2(gather_b0(by[h][0], by[h][1], by[h][2], by[h][3]),
                   gather_b0(by[h][4], by[h][5], by[h][6], by[h][7]));
}

template <int D>
__global__ void __launch_bounds__(2 * D) quantize_k_generic_kernel(
    const pnmix_page* __restrict__ jobs, const uint32_t* __restrict__ mask, int pairing, int n_hi,
    int G, int words, int bH, int bL) {
  __shared__ __align__(16) uint8_t lds[KWLds<D>::bytes];
  quantize_k_page_w<D>(jobs[blockIdx.x], mask, pairing, n_hi, G, words, bH, bL, lds);
}

template <int D, int BV>
__global__ void __launch_bounds__(2 * D) quantize_v_generic_kernel(const pnmix_page* __restrict__ jobs,
                                                                   int g_V) {
  __shared__ __align__(16) uint8_t lds[VWLds<D>::bytes];
  quantize_v_page_w<D, BV>(jobs[blockIdx.x], g_V, lds);
}

// key and value pages of any widths in one launch (workgroup 2i: key job i, 2i + 1: value job i)
template <int D, int BV>
__global__ void __launch_bounds__(2 * D) quantize_kv_generic_kernel(
    const pnmix_page* __restrict__ kjobs, const pnmix_page* __restrict__ vjobs,
    const uint32_t* __restrict__ mask, int pairing, int n_hi, int G, int words, int bH, int bL,
    int g_V) {
  constexpr int bytes = KWLds<D>::bytes > VWLds<D>::bytes ? KWLds<D>::bytes : VWLds<D>::bytes;
  __shared__ __align__(16) uint8_t lds[bytes];
  const int i = blockIdx.x >> 1;
  if (blockIdx.x & 1)
    quantize_v_page_w<D, BV>(vjobs[i], g_V, lds);
  else
    quantize_k_page_w<D>(kjobs[i], mask, pairing, n_hi, G, words, bH, bL, lds);
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
    hipLaunchKernelGGL(quantize_k_generic_kernel<DD>, dim3(n_pages), dim3(2 * DD), 0, stream, pages, \
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
#define PNMIX_QVW(DD, BB) \
  hipLaunchKernelGGL((quantize_v_generic_kernel<DD, BB>), dim3(n_pages), dim3(2 * DD), 0, stream, pages, c.g_V);
#define PNMIX_QV(DD)                                                                             \
  if (fast)                                                                                      \
    hipLaunchKernelGGL(quantize_v_kernel<DD>, dim3(n_pages), dim3(2 * DD), 0, stream, pages, c.g_V); \
  else if (c.b_V == 1) { PNMIX_QVW(DD, 1) }                                                      \
  else if (c.b_V == 4) { PNMIX_QVW(DD, 4) }                                                      \
  else { PNMIX_QVW(DD, 16) }
  switch (c.d) {
    case 32: PNMIX_QV(32) break;
    case 64: PNMIX_QV(64) break;
    default: PNMIX_QV(128) break;
  }
#undef PNMIX_QV
#undef PNMIX_QVW
  return hipGetLastError();
}

hipError_t launch_quantize_kv(const pnmix_cfg& c, int n_pages, const pnmix_page* kjobs,
                              const pnmix_page* vjobs, const uint32_t* mask, hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  const int words = (c.d / 2 + 31) / 32;
  const dim3 grid(2 * n_pages);
  if (!(c.b_H == 3 && c.b_L == 1 && c.b_V == 2)) {  // any other widths
#define PNMIX_QKVB(DD, BB)                                                                       \
    hipLaunchKernelGGL((quantize_kv_generic_kernel<DD, BB>), grid, dim3(2 * DD), 0, stream, kjobs,  \
                       vjobs, mask, c.pairing, c.n_hi_pairs, c.G, words, c.b_H, c.b_L, c.g_V);
#define PNMIX_QKVW(DD)                                                                           \
    if (c.b_V == 1) { PNMIX_QKVB(DD, 1) }                                                        \
    else if (c.b_V == 2) { PNMIX_QKVB(DD, 2) }                                                   \
    else if (c.b_V == 4) { PNMIX_QKVB(DD, 4) }                                                   \
    else { PNMIX_QKVB(DD, 16) }
    switch (c.d) {
      case 32: PNMIX_QKVW(32) break;
      case 64: PNMIX_QKVW(64) break;
      default: PNMIX_QKVW(128) break;
    }
#undef PNMIX_QKVW
#undef PNMIX_QKVB
    return hipGetLastError();
  }
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
