// quant_body.h -- device code of the page quantizers, shared by quant.hip (the page entry
// points) and prefill.hip (the fused prefill): the fp16 helpers, the Eq. 2 / Eq. 7 group
// metadata and code arithmetic, and the bodies of the register-tiled key and value page
// quantizers.  The file-level description of the algorithm is in quant.hip.
#pragma once

#include "common.h"
#include "kernels.h"

namespace pnmix {


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
// the single rounding of the fp32 subtraction), then the rest of code_bits.  Written out
// because the compiler turns fma(x, 1, c) into a conversion and a subtraction.  The compiler
// does not add wait states for an inline-asm consumer, so both operands must come from loads
// or plain VALU results (here: the loaded fp16 words and the negated group minimum), never
// straight from a transcendental instruction.
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


// page rows -> LDS [N][D] fp16
template <int D>
__device__ __forceinline__ void stage_page(uint16_t* xs, const uint16_t* src, int64_t stride) {
  for (int i = threadIdx.x; i < kN * D / 2; i += blockDim.x) {
    const int t = i / (D / 2), c2 = i % (D / 2);
    const uint16_t* r = src + (int64_t)t * stride + 2 * c2;
    reinterpret_cast<uint32_t*>(xs)[i] = (uint32_t)r[0] | ((uint32_t)r[1] << 16);
  }
}

}  // namespace pnmix
