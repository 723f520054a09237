// common.h -- device helpers shared by the gfx950 kernels of libpnmix.so.
//
// Build contract (see build.py): hipcc --offload-arch=gfx950 -O3 -ffp-contract=off, IEEE fp32
// division and square root (HIP's default correctly rounded expansion), fp16 denormals kept.
// Under these flags every float expression below is the IEEE operation it spells, so the
// quantizer and the score reproduce the reference arithmetic bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pnmix.h"

namespace pnmix {

constexpr int kWave = 64;
constexpr int kN = 128;  // page and residual length (tokens)

__device__ __forceinline__ float h2f(uint16_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, u));
}

// IEEE square root, round to nearest even, of a = 0, a normal float, +inf or NaN (no input
// below 2^-96 other than 0, so the hardware estimate needs no pre-scaling).  v_sqrt_f32 is
// within one ulp of the root r; the neighbours s - ulp and s + ulp decide: a <= (s - ulp) s
// puts r below the midpoint under s, a > (s + ulp) s above the midpoint over s (each residual
// one fma, exact enough to sign the difference).
__device__ __forceinline__ float sqrt_rn(float a) {
  const float s = __builtin_amdgcn_sqrtf(a);
  const float sd = __builtin_bit_cast(float, __builtin_bit_cast(int, s) - 1);
  const float su = __builtin_bit_cast(float, __builtin_bit_cast(int, s) + 1);
  const float vd = __builtin_fmaf(-sd, s, a);
  const float vu = __builtin_fmaf(-su, s, a);
  float r = vd <= 0.0f ? sd : s;
  r = vu > 0.0f ? su : r;
  return r;
}

// ||(x, y)|| of one RoPE pair of fp16 values in fp32: both squares are exact, their sum rounds
// once and the square root once (the same value as sqrtf(x * x + y * y) for finite x, y; the
// squares' sum is 0 or at least 2^-48).
__device__ __forceinline__ float pair_norm(uint16_t x, uint16_t y) {
  const float xf = h2f(x), yf = h2f(y);
  return sqrt_rn(__builtin_fmaf(xf, xf, __builtin_fmaf(yf, yf, 0.0f)));
}

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32 under the default rounding mode), with
// fp16 subnormals.
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

__device__ __forceinline__ float canon(float x) { return x + 0.0f; }  // -0 -> +0

// Mask bit of RoPE pair `pair` in a row of uint32 words (bit i = pair i, LSB first).
__device__ __forceinline__ bool pair_selected(const uint32_t* row, int pair) {
  return (row[pair >> 5] >> (pair & 31)) & 1u;
}

// Pair of channel `c` under the pairing: adjacent (2i, 2i+1) or split-half (i, i + d/2).
__device__ __forceinline__ int pair_of_channel(int c, int d, int pairing) {
  return pairing == PNMIX_PAIRS_ADJACENT ? (c >> 1) : (c < d / 2 ? c : c - d / 2);
}

// Rank of channel c among the salient channels in ascending channel order, or -1 when c is
// not salient (or its rank would reach 2 * n_hi).  Salient channels are both channels of every selected pair.
__device__ __forceinline__ int salient_rank(const uint32_t* row, int c, int d, int pairing,
                                            int n_hi) {
  const int p = pair_of_channel(c, d, pairing);
  if (!pair_selected(row, p)) return -1;
  int below = 0;  // selected pairs with index < p
  for (int w = 0; w < (p >> 5); ++w) below += __popc(row[w]);
  if (p & 31) below += __popc(row[p >> 5] & ((1u << (p & 31)) - 1u));
  const int r = pairing == PNMIX_PAIRS_ADJACENT ? 2 * below + (c & 1)
                                                : (c < d / 2 ? below : n_hi + below);
  // a mask with more than n_hi pairs set (outside the contract) must not index past the
  // n_sal columns of the upper-bit plane: such channels are treated as 1-bit
  return r < 2 * n_hi ? r : -1;
}

// Field of token t in a key bit plane of width w ([N/8][w][ncols] bytes): the w-bit fields of
// tokens 8j..8j+7 of one column form an 8w-bit little-endian stream, token 8j+k at bits
// wk..wk+w-1, stored as the w bytes [j][0..w-1] of that column (w = 1: the LSB byte of 8
// tokens; w = 2: two bytes of 4 tokens each, the PN-Mix kernel-implementation appendix).
__device__ __forceinline__ uint32_t plane_field(const uint8_t* plane, int ncols, int w, int col,
                                                int t) {
  const int j = t >> 3, pos = w * (t & 7), i0 = pos >> 3;
  const uint8_t* p = plane + (int64_t)(j * w + i0) * ncols + col;
  uint32_t v = p[0];
  if (i0 + 1 < w) v |= (uint32_t)p[ncols] << 8;
  return (v >> (pos & 7)) & ((1u << w) - 1u);
}

}  // namespace pnmix
