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

namespace pnmix {

constexpr int kN = 128;
constexpr int kOctets = kN / 8;
constexpr float kRound = 8388608.0f;  // 2^23

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u(half2_t h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
  return as_u(__builtin_elementwise_min(as_h2(a), as_h2(b)));
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  return as_u(__builtin_elementwise_max(as_h2(a), as_h2(b)));
}
__device__ __forceinline__ float lo_f(uint32_t u) { return h2f((uint16_t)(u & 0xffffu)); }
__device__ __forceinline__ float hi_f(uint32_t u) { return h2f((uint16_t)(u >> 16)); }
// bytes of a and b: (a.b0, b.b0, a.b1... ) helpers via v_perm_b32 (selector bytes 0-3 = b,
// 4-7 = a)
__device__ __forceinline__ uint32_t perm(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(a, b, sel);
}
// low bytes of four words -> one word (w0 in byte 0)
__device__ __forceinline__ uint32_t gather_b0(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const uint32_t p01 = perm(w1, w0, 0x0c0c0400u);  // [w0.b0, w1.b0, 0, 0]
  const uint32_t p23 = perm(w3, w2, 0x0c0c0400u);
  return perm(p23, p01, 0x05040100u);
}

// The 8 token rows 8k..8k+7, channels 8b..8b+7: x[j] = 8 fp16 of token 8k+j.
__device__ __forceinline__ void load_block(uint4 (&x)[8], const uint16_t* src, int64_t stride,
                                           int k, int b) {
  const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15) == 0) && ((stride & 7) == 0);
  const uint16_t* p = src + (int64_t)(8 * k) * stride + 8 * b;
  if (vec) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = *reinterpret_cast<const uint4*>(p + (int64_t)j * stride);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        w[m] = (uint32_t)p[(int64_t)j * stride + 2 * m] |
               ((uint32_t)p[(int64_t)j * stride + 2 * m + 1] << 16);
      x[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

__device__ __forceinline__ uint32_t word(const uint4& v, int m) {
  return m == 0 ? v.x : m == 1 ? v.y : m == 2 ? v.z : v.w;
}

// Eq. 2 / Eq. 7 metadata of one group with exact min mn and max mx; returns (mn, 1/s) with
// 1/s = 0 for a constant group (all codes then come out 0).
__device__ __forceinline__ float2 group_meta(float mn, float mx, int L, uint16_t& S,
                                             uint16_t& Z) {
  mn = canon(mn);
  mx = canon(mx);
  if (mx == mn) {
    S = 0;
    Z = f2h(mn);
    return make_float2(mn, 0.0f);
  }
  const float s = (mx - mn) / (float)L;
  const float inv = 1.0f / s;
  if (L == 1) {
    const float s7 = (mx - mn) * 0.5f;
    const float t3 = 3.0f * mn;
    const float z7 = (t3 + mx) * 0.25f;
    S = f2h(s7);
    Z = f2h(z7);
  } else {
    S = f2h(s);
    Z = f2h(mn);
  }
  return make_float2(mn, inv);
}

// Code of one element as the float 2^23 + q (q in the low mantissa bits).
__device__ __forceinline__ uint32_t code_bits(float x, float mn, float inv, float L) {
  const float y = (x - mn) * inv;
  return __float_as_uint(__builtin_amdgcn_fmed3f(y, 0.0f, L) + kRound);
}
// f16(low or high half of w) - mn in one v_fma_mix_f32 (w widened exactly, times 1, plus -mn:
// the single rounding of the fp32 subtraction), then the rest of code_bits.
__device__ __forceinline__ float sub_lo(uint32_t w, float nmn) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(nmn));
  return r;
}
__device__ __forceinline__ float sub_hi(uint32_t w, float nmn) {
  float r;
  asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(nmn));
  return r;
}
__device__ __forceinline__ uint32_t code_bits_h(uint32_t w, bool high, float nmn, float inv,
                                                float L) {
  const float y = (high ? sub_hi(w, nmn) : sub_lo(w, nmn)) * inv;
  return __float_as_uint(__builtin_amdgcn_fmed3f(y, 0.0f, L) + kRound);
}

// LDS of one key page: (min, max) fp16 per octet and channel, (min, 1/s) per group and
// channel, the upper-bit plane staging, the salient ranks.
template <int D>
struct KLds {
  static constexpr int part = 0;
  static constexpr int meta = part + kOctets * D * 4;
  static constexpr int hi = meta + (kN / 32) * D * 8;
  static constexpr int rank = hi + (kN / 4) * D;
  static constexpr int bytes = rank + D;
};

template <int D>
__device__ __forceinline__ void quantize_k_page(const pnmix_page& job,
                                                const uint32_t* __restrict__ mask, int pairing,
                                                int n_hi, int G, int words, uint8_t* lds) {
  constexpr int NB = D / 8;
  uint32_t* part = reinterpret_cast<uint32_t*>(lds + KLds<D>::part);
  float2* meta = reinterpret_cast<float2*>(lds + KLds<D>::meta);
  uint8_t* hi_s = lds + KLds<D>::hi;
  int8_t* rank_s = reinterpret_cast<int8_t*>(lds + KLds<D>::rank);
  const int tid = threadIdx.x, b = tid % NB, k = tid / NB;
  const int n_sal = 2 * n_hi;
  uint8_t* lo = job.dst;
  uint8_t* hi = lo + kN * D / 8;
  uint16_t* S = reinterpret_cast<uint16_t*>(hi + kN * n_sal / 4);
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
      pm[2 * m] = perm(mx, mn, 0x05040100u);      // channel 2m: (min.lo, max.lo)
      pm[2 * m + 1] = perm(mx, mn, 0x07060302u);  // channel 2m+1: (min.hi, max.hi)
    }
    uint4* dst = reinterpret_cast<uint4*>(part + k * D + 8 * b);
    dst[0] = make_uint4(pm[0], pm[1], pm[2], pm[3]);
    dst[1] = make_uint4(pm[4], pm[5], pm[6], pm[7]);
  }
  const uint32_t* mrow = mask + job.mask_row * words;
  if (tid < D) rank_s[tid] = (int8_t)salient_rank(mrow, tid, D, pairing, n_hi);
  __syncthreads();

  // B: one thread per (token group, channel)
  const int og = G / 8;  // octets per group
  for (int it = tid; it < (kN / G) * D; it += 2 * D) {
    const int g = it / D, c = it % D;
    float mn = lo_f(part[g * og * D + c]), mx = hi_f(part[g * og * D + c]);
    for (int o = 1; o < og; ++o) {
      const uint32_t v = part[(g * og + o) * D + c];
      mn = fminf(mn, lo_f(v));
      mx = fmaxf(mx, hi_f(v));
    }
    const int L = rank_s[c] >= 0 ? 7 : 1;
    uint16_t s, z;
    meta[g * D + c] = group_meta(mn, mx, L, s, z);
    S[g * D + c] = s;
    Z[g * D + c] = z;
  }
  __syncthreads();

  // C: codes of the thread's 8 channels x 8 tokens
  const int g = k / og;
  float2 mt[8];
  {
    const float4* src = reinterpret_cast<const float4*>(meta + g * D + 8 * b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = src[q];
      mt[2 * q] = make_float2(v.x, v.y);
      mt[2 * q + 1] = make_float2(v.z, v.w);
    }
  }
  int8_t rk[8];
  {
    const uint2 r = *reinterpret_cast<const uint2*>(rank_s + 8 * b);
#pragma unroll
    for (int s = 0; s < 8; ++s) rk[s] = (int8_t)(((s < 4 ? r.x : r.y) >> (8 * (s & 3))) & 0xff);
  }
  uint32_t lsb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int m = s >> 1;
    const float L = rk[s] >= 0 ? 7.0f : 1.0f;
    uint32_t u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u[j] = code_bits_h(word(x[j], m), (s & 1) != 0, -mt[s].x, mt[s].y, L);
    }
    // nibbles of tokens 0-3 and 4-7 in the low 16 bits (float exponent bits land >= bit 24)
    uint32_t wl = u[3], wh = u[7];
#pragma unroll
    for (int j = 2; j >= 0; --j) {
      wl = (wl << 4) | u[j];
      wh = (wh << 4) | u[j + 4];
    }
    const uint32_t nib = perm(wh, wl, 0x05040100u);  // token j in bits 4j..4j+2
    // LSB plane byte: bit j = code_j & 1
    uint32_t t = nib & 0x11111111u;
    t = (t | (t >> 3)) & 0x03030303u;
    t = (t | (t >> 6)) & 0x000f000fu;
    lsb[s] = t | (t >> 12);
    if (rk[s] >= 0) {
      // upper-bit plane: tokens 0-3 then 4-7, 2 bits each
      uint32_t h = (nib >> 1) & 0x33333333u;
      h = (h | (h >> 2)) & 0x0f0f0f0fu;
      h = (h | (h >> 4));
      hi_s[(2 * k) * n_sal + rk[s]] = (uint8_t)h;
      hi_s[(2 * k + 1) * n_sal + rk[s]] = (uint8_t)(h >> 16);
    }
  }
  {
    const uint32_t w0 = gather_b0(lsb[0], lsb[1], lsb[2], lsb[3]);
    const uint32_t w1 = gather_b0(lsb[4], lsb[5], lsb[6], lsb[7]);
    *reinterpret_cast<uint2*>(lo + k * D + 8 * b) = make_uint2(w0, w1);
  }
  __syncthreads();
  const int hi_chunks = (kN / 4) * n_sal / 16;
  for (int i = tid; i < hi_chunks; i += 2 * D)
    reinterpret_cast<uint4*>(hi)[i] = reinterpret_cast<const uint4*>(hi_s)[i];
}

template <int D>
__global__ void __launch_bounds__(2 * D) quantize_k_kernel(const pnmix_page* __restrict__ jobs,
                                                          const uint32_t* __restrict__ mask,
                                                          int pairing, int n_hi, int G,
                                                          int words) {
  __shared__ __align__(16) uint8_t lds[KLds<D>::bytes];
  quantize_k_page<D>(jobs[blockIdx.x], mask, pairing, n_hi, G, words, lds);
}

// Byte [m][t] of a value page holds channels 4m..4m+3 of token t (channel 4m+u in bits
// 2u..2u+1); the LDS copy of the code bytes keeps rows [m] of N bytes at a stride of kVRow
// words, which spreads the rows of one store over the banks.
constexpr int kVRow = kN / 4 + 2;

// LDS of one value page: (min, max) fp16 per token and 8-channel block, (min, 1/s) per token
// and group (<= 4), the page's code bytes [d/4][N] at a row stride of kVRow words.
template <int D>
struct VLds {
  static constexpr int part = 0;
  static constexpr int meta = part + kN * (D / 8) * 4;
  static constexpr int cw = meta + kN * 4 * 8;
  static constexpr int bytes = cw + (D / 4) * kVRow * 4;
};

template <int D>
__device__ __forceinline__ void quantize_v_page(const pnmix_page& job, int g_V, uint8_t* lds) {
  constexpr int NB = D / 8;
  uint32_t* part = reinterpret_cast<uint32_t*>(lds + VLds<D>::part);
  float2* meta = reinterpret_cast<float2*>(lds + VLds<D>::meta);
  uint32_t* cw = reinterpret_cast<uint32_t*>(lds + VLds<D>::cw);
  const int tid = threadIdx.x, b = tid % NB, k = tid / NB;
  const int ng = D / g_V;
  uint8_t* codes = job.dst;
  uint16_t* S = reinterpret_cast<uint16_t*>(codes + kN * D / 4);  // [ng][N]
  uint16_t* Z = S + kN * ng;                                        // [ng][N]

  uint4 x[8];
  load_block(x, job.src, job.src_row_stride, k, b);

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
  const int bg = g_V / 8;  // blocks per group
  for (int it = tid; it < kN * ng; it += 2 * D) {
    const int t = it % kN, gi = it / kN;
    const uint32_t* pr = part + t * NB + gi * bg;
    float mn = lo_f(pr[0]), mx = hi_f(pr[0]);
    for (int o = 1; o < bg; ++o) {
      mn = fminf(mn, lo_f(pr[o]));
      mx = fmaxf(mx, hi_f(pr[o]));
    }
    uint16_t s, z;
    meta[t * 4 + gi] = group_meta(mn, mx, 3, s, z);
    S[gi * kN + t] = s;
    Z[gi * kN + t] = z;
  }
  __syncthreads();

  // C: codes of the thread's 8 tokens x 8 channels.  Channels 8b..8b+3 and 8b+4..8b+7 are
  // byte columns 2b and 2b+1: each token's two bytes are formed here.  A code is the low byte
  // of its float 2^23 + q, so (u0 + 4 u1 + 16 u2 + 64 u3) has the byte q0 | q1 << 2 | q2 << 4 |
  // q3 << 6 in its low 8 bits (the exponent bits land above them).
  const int gi = b / bg;
  float2 mt[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mt[e] = meta[(8 * k + e) * 4 + gi];
  uint32_t by[2][8];  // [column 2b + i][token e], byte in bits 0..7
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t cu[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      cu[i] = code_bits_h(word(x[e], i >> 1), (i & 1) != 0, -mt[e].x, mt[e].y, 3.0f);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      by[h][e] = cu[4 * h] + (cu[4 * h + 1] << 2) + (cu[4 * h + 2] << 4) + (cu[4 * h + 3] << 6);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
    *reinterpret_cast<uint2*>(cw + (2 * b + h) * kVRow + 2 * k) =
        make_uint2(gather_b0(by[h][0], by[h][1], by[h][2], by[h][3]),
                   gather_b0(by[h][4], by[h][5], by[h][6], by[h][7]));
  __syncthreads();
  // 16-byte pieces of the code area, one per thread: row tid / 8, bytes 16 (tid % 8) ..
  {
    const uint32_t* src = cw + (tid / 8) * kVRow + 4 * (tid % 8);
    const uint2 lo2 = *reinterpret_cast<const uint2*>(src);
    const uint2 hi2 = *reinterpret_cast<const uint2*>(src + 2);
    reinterpret_cast<uint4*>(codes)[tid] = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
  }
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

// page rows -> LDS [N][D] fp16
template <int D>
__device__ __forceinline__ void stage_page(uint16_t* xs, const uint16_t* src, int64_t stride) {
  for (int i = threadIdx.x; i < kN * D / 2; i += blockDim.x) {
    const int t = i / (D / 2), c2 = i % (D / 2);
    const uint16_t* r = src + (int64_t)t * stride + 2 * c2;
    reinterpret_cast<uint32_t*>(xs)[i] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
  }
}

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
