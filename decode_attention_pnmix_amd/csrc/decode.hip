// decode.hip -- split-K GQA decode attention straight over the PN-Mix packed cache (gfx950).
//
// PN-Mix paper (arXiv 2610.19605), sec. 2, Eq. 1: causal GQA softmax attention at the decode
// position; kernel-implementation appendix: each step visits the sink region, the quantized
// region and the residual region, and the dequantized cache is never written back (each packed
// group is unpacked on chip and consumed at once).  TriAxialKV fact sheet: flash-decoding
// splits merged by online log-sum-exp.
//
// Work decomposition.  One wave takes one (sequence, KV head, split); a workgroup holds one wave
// or (for small batches) up to eight, whose partials it merges on chip.  A page split walks a
// run of packed pages; the fp16 splits take 64-token chunks of the sink and residual rows.  All
// n_g query heads of the GQA group are served from one read of each page, so every packed byte
// crosses HBM once per step.  Partials (m, l, o) in log2 units go to the workspace; a second
// kernel merges them.
//
// Page split, per page (keys quantized per channel, k = S_c q + Z_c; values per token and group,
// v = S_tg q + Z_tg):
//   logit(h, t) = sum_c (qt_hc S_c) code_tc + sum_c qt_hc Z_c,   qt = q * sm_scale * log2(e)
//   o(h, c)    += sum_t (p_ht S_tg) code_tc + sum_t p_ht Z_tg
// * q.K runs on the int8 matrix cores (v_mfma_i32_16x16x64_i8).  The per-page products
//   qt_hc S_c become 32-bit fixed point (one power-of-two scale per page for the GQA group,
//   from the group's max|qt| and the page's max S) and are split into four signed base-256
//   digits: rows of the A operand are (head, digit), columns of the B operand are 16 keys, K is
//   64 channels.  The B operand is the packed code itself: the
//   LSB plane byte of (channel, 8 tokens) and the upper-bit plane byte of (salient channel,
//   4 tokens) are masked in place, one bit field per MFMA, so a tile holds the keys 8i + b of a
//   page (i = 0..15) and a 16-byte load of either plane feeds eight tiles.  The upper-bit rows
//   hold the LSB rows' digit words of the salient channels, written by the same per-page loop at
//   each channel's salient rank.  Integer accumulation is exact; the four digit partials of a
//   key sit in one lane and are combined in fp32.
// * p.V runs on the int8 matrix cores too.  w = p S_tg per (head, key, value group) becomes
//   fixed point below 2^22 with a per-head power-of-two scale set from that head's largest p on
//   the page times the page's largest value scale (so the result does not depend on how pages
//   are split); its three base-256 digits (the two lower ones balanced, in [-128, 127]) go to an
//   LDS table whose rows are (head, digit).  The B operand is again the packed value byte
//   masked in place.  A byte holds 4 consecutive channels of one token (byte column m =
//   channels 4m..4m+3, the N tokens of a column contiguous), so a tile takes 8 byte columns
//   (32 channels, inside one value group of g_V >= 32) and two of their four 2-bit fields:
//   column n < 8 reads byte column n with field f, column n >= 8 byte column n - 8 with field
//   f + 2.  The 16 bytes a lane loads for its column serve two tiles (f = 0 and f = 1).
// * The Z terms and the softmax bookkeeping run on the vector ALU in fp32.
#include <algorithm>

#include "common.h"
#include "decode_args.h"
#include "kernels.h"

namespace pnmix {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kMergeSplits = 136;
constexpr long long kPieceCost = 5;  // planner cost of a 32-token fp16 piece on a page wave (a page: 4)  // the planner's cap: beyond it the merge costs more than it saves
constexpr int kWS = kN + 16;     // row stride of the p.V digit table (rows on distinct banks)
constexpr float kLog2e = 1.4426950408889634f;
// y + 2^23 + 0x8080 rounds y in [0, 2^23 - 0x8080) to an integer (RNE) and leaves y + 0x8080
// in the low 23 bits of the float: bytes 0 and 1 xor 0x80 are y's balanced base-256 digits
constexpr float kTwo23b = 8421504.0f;


template <int D, int KH>
struct Shape {
  static constexpr int KL = (D + 63) / 64;   // 64-channel K-steps over the LSB plane
  static constexpr int KHM = KH;             // 64-rank K-steps over the upper-bit plane
  // bytes per (head, digit) row of the q.K digit table: 64 per K-step, plus 16 so that the
  // 16 rows of an A-operand read start on 16 different 4-bank groups
  static constexpr int TL = 64 * (KL + KHM) + 16;
  static constexpr int JL = D / 4;           // 4-channel units per head
};

// ---------------------------------------------------------------------------- small helpers

// Lane permutations inside a 16-lane row.  Every pattern used here (quad_perm, row_ror,
// row_half_mirror) reads a valid lane for every lane, so bound_ctrl never applies; setting it
// lets the compiler fold the move into the consuming add or integer max (one instruction per
// step).
template <int CTRL>
__device__ __forceinline__ float dpp_c(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, true));
}
// all-reduce over the 16 lanes of a row (lanes 16r .. 16r+15)
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp_c<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_c<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_c<0x124>(x));  // row_ror:4
  x = fmaxf(x, dpp_c<0x128>(x));  // row_ror:8
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x = x + dpp_c<0xB1>(x);
  x = x + dpp_c<0x4E>(x);
  x = x + dpp_c<0x124>(x);
  x = x + dpp_c<0x128>(x);
  return x;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}
// Across the four 16-lane rows: the row results are read into scalar registers (v_readlane)
// and combined there, with no LDS round trip.  rowv(x, r) = x of row r (x uniform per row).
__device__ __forceinline__ float rowv(float x, int r) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16 * r));
}
__device__ __forceinline__ float row_sum_all16(float x) {  // x: row all-reduced
  x = x + dpp_c<0xB1>(x);
  x = x + dpp_c<0x4E>(x);
  x = x + dpp_c<0x124>(x);
  return x + dpp_c<0x128>(x);
}
__device__ __forceinline__ float row_max_all16(float x) {
  x = fmaxf(x, dpp_c<0xB1>(x));
  x = fmaxf(x, dpp_c<0x4E>(x));
  x = fmaxf(x, dpp_c<0x124>(x));
  return fmaxf(x, dpp_c<0x128>(x));
}

// all-reduce over aligned groups of W lanes (W a power of two, 8 <= W <= 64)
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  if (W == 8) {
    x = x + dpp_c<0xB1>(x);
    x = x + dpp_c<0x4E>(x);
    return x + dpp_c<0x141>(x);  // row_half_mirror: lane i and 7 - i of each 8
  }
  x = row_sum_all16(x);
  if (W == 16) return x;
  const float h0 = rowv(x, 0) + rowv(x, 1), h1 = rowv(x, 2) + rowv(x, 3);
  if (W == 32) return threadIdx.x % 64 < 32 ? h0 : h1;
  return h0 + h1;
}
template <int W>
__device__ __forceinline__ float group_max(float x) {
  if (W == 8) {
    x = fmaxf(x, dpp_c<0xB1>(x));
    x = fmaxf(x, dpp_c<0x4E>(x));
    return fmaxf(x, dpp_c<0x141>(x));
  }
  x = row_max_all16(x);
  if (W == 16) return x;
  const float h0 = fmaxf(rowv(x, 0), rowv(x, 1)), h1 = fmaxf(rowv(x, 2), rowv(x, 3));
  if (W == 32) return threadIdx.x % 64 < 32 ? h0 : h1;
  return fmaxf(h0, h1);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u<0xB1>(x));
  x = max(x, dpp_u<0x4E>(x));
  x = max(x, dpp_u<0x124>(x));
  x = max(x, dpp_u<0x128>(x));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(r0, r1), max(r2, r3));
}
// maximum over the wave of non-negative floats (their bit patterns order like the values)
__device__ __forceinline__ float wave_max_nonneg(float x) {
  return __builtin_bit_cast(float, wave_max_u32(__builtin_bit_cast(uint32_t, x)));
}

__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
// two fp32 -> packed fp16, round to nearest even (v_cvt_pk_f16_f32): the lo half of a split
// then carries no same-sign rounding bias even where it falls into the fp16 subnormal range
__device__ __forceinline__ uint32_t pk_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, v2h{(_Float16)a, (_Float16)b});
}
__device__ __forceinline__ float pow2i(int e) {  // 2^e for e in [-126, 127]
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}
__device__ __forceinline__ float sel4(const v4f& v, int i) {
  float r = v[0];
  r = i == 1 ? v[1] : r;
  r = i == 2 ? v[2] : r;
  r = i == 3 ? v[3] : r;
  return r;
}

// Balanced base-256 digits of x (|x| < 2^30): byte d of the result, read as int8, is digit d
// and x = sum_d 256^d digit_d.
__device__ __forceinline__ uint32_t digits4(int x) {
  return ((uint32_t)x + 0x80808080u) ^ 0x80808080u;
}
// sum_d 256^d c[d] of four int32 digit partial sums, in fp32 (c[0] + 256 c[1] and
// c[2] + 256 c[3] are formed exactly in int32 first: each |c[d]| < 2^22)
__device__ __forceinline__ float combine4(const v4i& c) {
  const int lo = c[0] + (c[1] << 8), hi = c[2] + (c[3] << 8);
  return __builtin_fmaf((float)hi, 65536.0f, (float)lo);
}
// a * f16(low or high half of h) + c with one rounding (the fp16 operand widens exactly); the
// compiler selects v_fma_mix_f32 for it and keeps track of its hazards (an inline-asm form
// would not get the wait state a transcendental result needs before its use)
__device__ __forceinline__ float fma_mix_lo(float a, uint32_t h, float c) {
  return __builtin_fmaf(a, f16lo(h), c);
}
__device__ __forceinline__ float fma_mix_hi(float a, uint32_t h, float c) {
  return __builtin_fmaf(a, f16hi(h), c);
}
typedef uint16_t v2u16 __attribute__((ext_vector_type(2)));
// packed max of two pairs of non-negative fp16 values through their bit patterns (which order
// like the values), without the NaN canonicalisation of a floating-point max
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(v2u16, a),
                                                                __builtin_bit_cast(v2u16, b)));
}
// sum_t x_t B_t from the p.V digit sums: c[0], c[1] of the balanced low digits, c[2] of the
// top digit (c[3], the fourth row of each head, is not used); c[0] + 256 c[1] is exact in
// int32 (|c[d]| < 2^20)
__device__ __forceinline__ float combine_pv(const v4i& c) {
  const int lo = c[0] + (c[1] << 8);
  return __builtin_fmaf((float)c[2], 65536.0f, (float)lo);
}
// bytes 0..2 of four words, transposed: out[d] byte i = byte d of y[i]
__device__ __forceinline__ void transpose3(const uint32_t y[4], uint32_t out[3]) {
  const uint32_t t0 = __builtin_amdgcn_perm(y[1], y[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(y[1], y[0], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(y[3], y[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(y[3], y[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
}
// 4 x 4 byte transpose: out[d] byte i = byte d of y[i]
__device__ __forceinline__ void transpose4(const uint32_t y[4], uint32_t out[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(y[1], y[0], 0x05010400u);
  const uint32_t t1 = __builtin_amdgcn_perm(y[1], y[0], 0x07030602u);
  const uint32_t t2 = __builtin_amdgcn_perm(y[3], y[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(y[3], y[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Key codes of tile b as int8 B-operand bytes.  Tile b holds token 8i + b of octet i (LSB plane
// bit b; upper-bit plane row 2i + b/4, field b%4).  Each field is masked in place, scaled by
// sL(b) for the LSB and sH(b) = 2 sL(b) for the upper bits (their weight in the code is 2), so
// one accumulator holds sL(b) * sum digit * code.
template <int B>
__device__ __forceinline__ uint32_t lsb_field(uint32_t w) {
  if (B <= 4) return w & (0x01010101u << B);
  if (B == 5) return (w >> 4) & 0x02020202u;
  if (B == 6) return (w >> 3) & 0x08080808u;
  return (w >> 4) & 0x08080808u;
}
template <int B>
__device__ __forceinline__ uint32_t hi_field(uint32_t w) {
  if (B == 0) return (w << 1) & 0x06060606u;
  if (B == 1) return w & 0x0C0C0C0Cu;
  if (B == 2) return (w >> 1) & 0x18181818u;
  if (B == 3) return (w >> 2) & 0x30303030u;
  if (B == 4) return (w << 5) & 0x60606060u;
  if (B == 5) return w & 0x0C0C0C0Cu;
  if (B == 6) return w & 0x30303030u;
  return (w >> 2) & 0x30303030u;
}
__device__ constexpr float kInvSL[8] = {1.0f, 0.5f, 0.25f, 0.125f, 0.0625f, 0.5f, 0.125f, 0.125f};

// Buffer loads: one resource per (sequence, KV head) cache, a wave-uniform page offset in an
// SGPR and loop-invariant lane offsets, so a page costs no per-lane address arithmetic.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buf_rsrc(const void* base, int64_t bytes) {
  const int n = (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ v4u bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v[0], v[1]);
}
// 16 bytes at any offset, in two steps so that no wait sits between them: the five aligned
// dwords that cover them (bload20) and, where the bytes are consumed, the byte shift (align20)
struct Raw20 {
  uint32_t d[5];
};
__device__ __forceinline__ Raw20 bload20(rsrc_t r, uint32_t voff, uint32_t soff) {
  Raw20 x;
#pragma unroll
  for (int i = 0; i < 5; ++i) x.d[i] = __builtin_amdgcn_raw_buffer_load_b32(r, (voff & ~3u) + 4 * i, soff, 0);
  return x;
}
__device__ __forceinline__ v4u align20(const Raw20& x, uint32_t voff) {
  const uint32_t sh = voff & 3u;
  return v4u{__builtin_amdgcn_alignbyte(x.d[1], x.d[0], sh), __builtin_amdgcn_alignbyte(x.d[2], x.d[1], sh),
             __builtin_amdgcn_alignbyte(x.d[3], x.d[2], sh), __builtin_amdgcn_alignbyte(x.d[4], x.d[3], sh)};
}
// Wave-uniform data that the kernel never writes (cache lengths, pair mask), read through the
// constant address space so that it arrives by scalar loads, which a wait for vector loads
// does not cover.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* kconst(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}
// 16 bytes at a 2-byte-aligned offset: five aligned dwords and a byte shift
__device__ __forceinline__ v4u bload16_a2(rsrc_t r, uint32_t voff, uint32_t soff) {
  const uint32_t a = voff & ~3u, sh = voff & 3u;
  uint32_t d[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) d[i] = __builtin_amdgcn_raw_buffer_load_b32(r, a + 4 * i, soff, 0);
  v4u out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = sh ? __builtin_amdgcn_alignbyte(d[i + 1], d[i], sh) : d[i];
  return out;
}

// ------------------------------------------------------------------------- partial writers

// LDS hand-off between the lanes of one wave.  Every wave owns its slice of LDS and the LDS unit
// executes one wave's instructions in order, so waiting for the wave's own LDS operations plus a
// compiler barrier orders them; no workgroup barrier is involved, and the waves of a workgroup
// run their splits independently.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt left open
  __asm__ volatile("" ::: "memory");
}

// Where a split leaves its partial: o [n_g][d] and (m, l) [n_g][2], in the workspace (one wave
// per workgroup) or in the wave's LDS slice for the workgroup's own merge.  Both are stored
// through typed pointers (global or LDS instructions): a store through a generic pointer is a
// FLAT instruction, and one in flight on any path makes the compiler wait for every load in
// flight at the next use of a loaded value.
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) v4f lds_v4f;
struct PartOut {
  float* go;    // workspace o and (m, l), or
  float* gml;
  lds_f32* lo;  // the LDS slice's o and (m, l) when in_lds
  lds_f32* lml;
  bool in_lds;
  __device__ __forceinline__ void o(int i, float v) const {
    if (in_lds) lo[i] = v; else go[i] = v;
  }
  __device__ __forceinline__ void o4(int i, const v4f& v) const {
    if (in_lds) *reinterpret_cast<lds_v4f*>(lo + i) = v;
    else *reinterpret_cast<v4f*>(go + i) = v;
  }
  __device__ __forceinline__ void ml(int hh, float m, float l) const {
    if (in_lds) {
      lml[2 * hh] = m;
      lml[2 * hh + 1] = l;
    } else {
      gml[2 * hh] = m;
      gml[2 * hh + 1] = l;
    }
  }
};

template <int D>
__device__ void write_empty_partial(const DecodeArgs& a, const PartOut& po) {
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < a.n_g * D; i += 64) po.o(i, 0.0f);
  if (lane < a.n_g) po.ml(lane, -INFINITY, 0.0f);
}

// -------------------------------------------------------------- fp16 sink + residual split

// V^T staging of the fp16 rows in a wave's LDS slice: [D][32 tokens + 4] halves (the pad spreads
// the banks)
template <int D>
constexpr int kVtBytes = D * 36 * 2;

// One wave over the 32-token pieces first, first + stride, ... of the fp16 rows (token order:
// sinks, then residual rows) on the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16, exact fp16 products, fp32 sums):
// * logits transposed, S^T[token][head] = K q^T: the A operand is the key rows as loaded (16
//   bytes of one token per lane), the B operand the queries (head = lane column);
// * lane (g, n) of the S^T result holds head n for tokens 4g + r and 16 + 4g + r, r < 4.  With
//   the 32 tokens of the reduction numbered in that order, this is the B operand of
//   O^T = V^T P^T, so p never leaves its lane; it enters as fp16 hi + lo (two MFMAs, ~22 bits);
// * V^T comes from LDS: 16-byte loads of 4 value rows are transposed with byte permutes into
//   [channel][token] rows;
// * every softmax quantity of head n lives in the lanes of column n: the maximum is taken over
//   the lane's 8 tokens, then over the four lane groups.
// t_new >= 0: fp16 row t_new (sinks first, then residual rows) is the fused append's new row,
// read from k_new / v_new instead of the cache.
// mo != NULL: the same wave's page partial (o [n_g][D], then (m, l) [n_g][2]) is in LDS at mo;
// it is merged into this partial (log-sum-exp rule) before the store.
template <int D>
__device__ void fp16_region(const DecodeArgs& a, int b, int h, int64_t bh, const PartOut& po,
                            int sink_len, int res_len, int first, int stride, uint8_t* lds,
                            int t_new, const lds_f32* mo) {
  constexpr int KS = D / 32;         // 32-channel K-steps of S^T
  constexpr int CT = D / 16;         // 16-channel tiles of O^T
  constexpr int VS = kVtBytes<D> / (2 * D);  // V^T row stride in halves: 32 tokens + 4
  constexpr int OC = D / 8;          // 8-channel pieces of a row
  constexpr int VU = (8 * OC + 63) / 64;  // (4 tokens x 8 channels) staging units per lane
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int ng = a.n_g;
  uint16_t* vT = reinterpret_cast<uint16_t*>(lds);  // [D][VS]
  const int T16 = sink_len + res_len;
  // No branches around loads (a wait would sit in each): the queries come by buffer loads
  // (heads past n_g read as zero), and a token past the fp16 rows reads the last row instead,
  // whose logit is then masked to -inf and whose p is 0 (finite values times 0).
  const rsrc_t qrs = buf_rsrc(a.q + ((int64_t)b * a.H_q + (int64_t)h * ng) * D, (int64_t)ng * D * 2);
  v4u qv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qv[ks] = bload16(qrs, (uint32_t)(2 * (n * D + 32 * ks + 8 * g)), 0u);
  const uint16_t* k_s = a.k_sink + bh * a.N_s * D;
  const uint16_t* v_s = a.v_sink + bh * a.N_s * D;
  const uint16_t* k_r = a.k_res + bh * kN * D - (int64_t)sink_len * D;  // row t >= sink_len
  const uint16_t* v_r = a.v_res + bh * kN * D - (int64_t)sink_len * D;
  const uint16_t* k_n = t_new >= 0 ? a.k_new + bh * D : k_s;
  const uint16_t* v_n = t_new >= 0 ? a.v_new + bh * D : v_s;
  auto krow = [&](int t) {
    t = min(t, T16 - 1);
    return t == t_new ? k_n : (t < sink_len ? k_s : k_r) + (int64_t)t * D;
  };
  auto vrow = [&](int t) {
    t = min(t, T16 - 1);
    return t == t_new ? v_n : (t < sink_len ? v_s : v_r) + (int64_t)t * D;
  };
  float m = -INFINITY, l = 0.0f;  // l: this lane's tokens only, summed over lane groups at the end
  v4f acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // this wave's 32-token pieces; the loads of the next piece are issued before the current one
  // is computed
  auto s0_of = [&](int k) { return 32 * (first + k * stride); };
  auto load_piece = [&](int s0, v4u (&ka)[2][KS], v4u (&vr)[VU][4]) {
    // key rows (A of S^T): tile tt holds tokens s0 + 16 tt + n, channels 32 ks + 8 g ...
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint16_t* row = krow(s0 + 16 * tt + n);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[tt][ks] = *reinterpret_cast<const v4u*>(row + 32 * ks + 8 * g);
    }
    // value rows: unit u = tokens s0 + 4 (u / OC) + 0..3, channels 8 (u % OC) + 0..7
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = lane + 64 * j;
      const int tq = u / OC, oc = u % OC;
#pragma unroll
      for (int i = 0; i < 4; ++i)  // (lanes past the units read a valid row; it is not stored)
        vr[j][i] = *reinterpret_cast<const v4u*>(vrow(s0 + 4 * tq + i) + 8 * (oc % OC));
    }
  };
  // one 32-token piece: S^T, V^T to LDS, online softmax, O^T += V^T P^T
  auto piece = [&](int s0, const v4u (&ka)[2][KS], const v4u (&vr)[VU][4]) {
    v4f st[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      st[tt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        st[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, ka[tt][ks]),
                                                        __builtin_bit_cast(v8h, qv[ks]), st[tt], 0, 0, 0);
    }
    // V^T: channel 8 oc + c, tokens 4 tq .. 4 tq + 3 as one 8-byte row piece
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = lane + 64 * j;
      if (u < 8 * OC) {
        const int tq = u / OC, oc = u % OC;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w0 = vr[j][0][e], w1 = vr[j][1][e], w2 = vr[j][2][e], w3 = vr[j][3][e];
          *reinterpret_cast<uint2*>(vT + (8 * oc + 2 * e) * VS + 4 * tq) =
              make_uint2(__builtin_amdgcn_perm(w1, w0, 0x05040100u), __builtin_amdgcn_perm(w3, w2, 0x05040100u));
          *reinterpret_cast<uint2*>(vT + (8 * oc + 2 * e + 1) * VS + 4 * tq) =
              make_uint2(__builtin_amdgcn_perm(w1, w0, 0x07060302u), __builtin_amdgcn_perm(w3, w2, 0x07060302u));
        }
      }
    }
    // online softmax of head n over the 32 tokens (log2 units)
    float sv[8];
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = s0 + 16 * (i >> 2) + 4 * g + (i & 3);
      sv[i] = t < T16 ? st[i >> 2][i & 3] * a.qscale : -INFINITY;
      cm = fmaxf(cm, sv[i]);
    }
    cm = fmaxf(cm, __shfl_xor(cm, 16));
    cm = fmaxf(cm, __shfl_xor(cm, 32));  // finite: token s0 is valid
    const float mn = fmaxf(m, cm);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    float p[8], ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(sv[i] - mn);
      ps += p[i];
    }
    l = l * alpha + ps;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] *= alpha;
    v4u phi, plo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      phi[e] = pk_rne(p[2 * e], p[2 * e + 1]);
      plo[e] = pk_rne(p[2 * e] - f16lo(phi[e]), p[2 * e + 1] - f16hi(phi[e]));
    }
    wave_sync();  // V^T is in LDS
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const uint16_t* vrow = vT + (16 * ct + n) * VS;
      const uint2 x0 = *reinterpret_cast<const uint2*>(vrow + 4 * g);
      const uint2 x1 = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * g);
      const v8h va = __builtin_bit_cast(v8h, v4u{x0.x, x0.y, x1.x, x1.y});
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, __builtin_bit_cast(v8h, phi), acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, __builtin_bit_cast(v8h, plo), acc[ct], 0, 0, 0);
    }
    wave_sync();  // V^T is rewritten by the next 32 tokens
  };
  // two register sets, each loaded one piece ahead of its use (no copies between them)
  v4u ka0[2][KS], vr0[VU][4], ka1[2][KS], vr1[VU][4];
  if (s0_of(0) < T16) {
    load_piece(s0_of(0), ka0, vr0);
    // (the next piece is loaded unconditionally, rows clamped to the last one: no load sits
    // under a branch)
    for (int k = 0;; k += 2) {
      load_piece(s0_of(k + 1), ka1, vr1);
      piece(s0_of(k), ka0, vr0);
      if (s0_of(k + 1) >= T16) break;
      load_piece(s0_of(k + 2), ka0, vr0);
      piece(s0_of(k + 1), ka1, vr1);
      if (s0_of(k + 2) >= T16) break;
    }
  }
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (mo) {
    wave_sync();  // the page partial is in LDS
    if (n < ng) {
      const lds_f32* mml = mo + ng * D;
      const float mp = mml[2 * n], lp = mml[2 * n + 1];
      const float M = fmaxf(m, mp);
      const float f1 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      const float f2 = mp == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mp - M);
      l = __builtin_fmaf(lp, f2, l * f1);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v4f op = *reinterpret_cast<const lds_v4f*>(mo + n * D + 16 * ct + 4 * g);
        acc[ct] = acc[ct] * f1 + op * f2;
      }
      m = M;
    }
  }
  if (n < ng) {
    // O^T: lane (g, n) holds channels 16 ct + 4 g + r of head n
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      po.o4(n * D + 16 * ct + 4 * g, acc[ct]);
    if (g == 0) po.ml(n, m, l);
  }
}

// The fp16 rows of (sequence, KV head) bh, 32-token pieces first, first + stride, ...: the
// lengths (with a fused append's new row) and then fp16_region.
template <int D>
__device__ __forceinline__ void fp16_split(const DecodeArgs& a, int64_t bh, const PartOut& po, int first,
                                           int stride, uint8_t* wl, const lds_f32* mo) {
  const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
  pnmix_seq_len L;
  L.sink_len = kconst(&a.lens[b].sink_len)[0];
  L.n_pages = kconst(&a.lens[b].n_pages)[0];
  L.res_len = kconst(&a.lens[b].res_len)[0];
  int t_new = -1;
  if (a.k_new) {  // the fused append's row joins the fp16 rows
    int kind, row;
    append_slot(L, a.N_s, kind, row);
    if (kind == 0) L.sink_len = row + 1;
    if (kind == 1) L.res_len = row + 1;
    if (kind != 2) t_new = kind == 0 ? row : min(max(L.sink_len, 0), a.N_s) + row;
  }
  const int sink_len = min(max(L.sink_len, 0), a.N_s);
  const int res_len = min(max(L.res_len, 0), kN);
  fp16_region<D>(a, b, h, bh, po, sink_len, res_len, first, stride, wl, t_new, mo);
}

// ----------------------------------------------------------------------------- page split

// Rank of channel c among the salient channels (-1 if not salient) from the first two words of
// the pair mask held in registers (d <= 128: at most 64 pairs).  Same ranking as the packer:
// ascending pair index; adjacent pairs interleave their two channels, half-split pairs list the
// first halves, then the second halves.
__device__ __forceinline__ int salient_rank2(uint32_t w0, uint32_t w1, int c, int d, int pairing,
                                             int n_hi) {
  const int p = pair_of_channel(c, d, pairing);
  const uint64_t mk = (uint64_t)w0 | ((uint64_t)w1 << 32);
  if (!((mk >> p) & 1u)) return -1;
  const int below = __popcll(mk & ((1ull << p) - 1ull));
  const int r = pairing == PNMIX_PAIRS_ADJACENT ? 2 * below + (c & 1)
                                                : (c < d / 2 ? below : n_hi + below);
  return r < 2 * n_hi ? r : -1;
}

template <int D, int NT, int KG, int KH, bool PG>
__device__ void page_split(const DecodeArgs& a, uint8_t* lds, int split, int64_t bh,
                           const PartOut& po) {
  using S_ = Shape<D, KH>;
  constexpr int KL = S_::KL, KHM = S_::KHM, TL = S_::TL, JL = S_::JL;
  constexpr int NH = 4 * NT;
  constexpr int UK = (NT * D + 63) / 64;   // LSB prep units per lane
  constexpr int NTV = D / 16;              // p.V column tiles of 16 channels
  constexpr int NBLK = D / 32;             // blocks of 8 value-byte columns (32 channels)
  // Both sides of the next page are fetched a page ahead (the keys once q.K is done, the
  // values once p.V is done) where that fits in registers: one head tile, or two with one key
  // group.  Elsewhere the values are fetched after q.K and the next keys after p.V.
  constexpr bool kLate = !(NT == 1 || (NT == 2 && KG == 1));

  const int lane = threadIdx.x & 63;
  const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
  const int ng = a.n_g;
  const int G = a.G, n_sal = a.n_sal, NGV = a.NGV;
  // The queries and the first page do not depend on the cache lengths: their loads go first,
  // the queries ahead of the page (a wait for them must not wait for the page).
  // LSB prep units: unit u = lane + 64k -> head hu = u / JL (0..NH-1), channels 4 (u % JL) + 0..3
  // (buffer loads: heads past the group's n_g read as zero, with no branch to wait in)
  const rsrc_t qrs = buf_rsrc(a.q + ((int64_t)b * a.H_q + (int64_t)h * ng) * D, (int64_t)ng * D * 2);
  uint2 qq[UK];
#pragma unroll
  for (int k = 0; k < UK; ++k) {
    const int u = lane + 64 * k;
    qq[k] = bload8(qrs, (uint32_t)(2 * 4 * u), 0u);  // head u / JL, channels 4 (u % JL) + 0..3
  }
  const int oct = lane & 15;  // octet of the q.K B operand (keys 8 oct + b)
  const int qb = lane >> 4;   // K block (16 channels / 8 keys) of this lane
  const int kg_lane = (8 * oct) / G;  // key group of this lane's keys
  const int sOff = kN * D / 8 + kN * n_sal / 4;      // K page: S after lo and hi planes
  const int zOff = sOff + 2 * KG * D;
  // p.V: this lane's value-byte column within a block of 8, and its B-operand mask: field 0
  // (column n < 8) or field 2 (n >= 8) of every byte in place, for the tiles of field pair
  // (0, 2); the tiles of pair (1, 3) mask the bytes shifted right by 2 the same way.  Field 2
  // in place weighs 16 (codes 0..48: no int8 sign bit), so the lane's weight is 1 or 1/16.
  const int vcol = lane & 7;
  const uint32_t vmask = (lane & 8) ? 0x30303030u : 0x03030303u;
  const float vfw = (lane & 8) ? 0.0625f : 1.0f;

  // Key side of one page in registers: this lane's packed codes (LSB rows and upper-bit rows
  // 2 oct, 2 oct + 1) and the scales of its prep units.  The next page's are loaded into them as
  // soon as the current page's q.K is done, so their latency hides behind softmax and p.V.
  v4u wL[KL];
  Raw20 hr0[KHM], hr1[KHM];  // upper-bit rows as loaded (any byte alignment)
  // 4 fp16 of S and Z per key group for this lane's channels 4 j .. 4 j + 3, j = lane % JL
  // (the same channels for every prep unit of the lane: 64 is a multiple of JL)
  uint2 sv[KG], zv[KG];
  // Contiguous pages [B][max_pages][H_kv][bytes] (the block pool's layout, block b * max_pages
  // + p): page pg of this head lies pg * H_kv * bytes past this head's first page
  const int64_t page_row = ((int64_t)b * a.max_pages * a.H_kv + h);
  const int64_t span = ((int64_t)(a.max_pages - 1) * a.H_kv + 1);
  const rsrc_t krs = buf_rsrc(a.k_pages + page_row * a.kpb, a.max_pages > 0 ? span * a.kpb : 0);
  const rsrc_t vrs = buf_rsrc(a.v_pages + page_row * a.vpb, a.max_pages > 0 ? span * a.vpb : 0);
  // The next page's loads are issued whether or not there is a next page, through a resource
  // of zero bytes when there is none (every lane reads zero, nothing is fetched): a load under
  // a branch would make the compiler wait, on the path that issued it, for everything in flight
  // wherever an older load's data is used after the branch rejoins.
  const rsrc_t nul = buf_rsrc(a.k_pages, 0);
  // Page pg of this (sequence, KV head): contiguous pages share one resource at offset
  // pg * H_kv * bytes; with a block table the page is block table[b][pg] of the pool (its own
  // resource, offset 0; the block index is clamped to the pool, so no entry can address
  // outside it).
  // The block of page pg (table entries are read once per page, ahead of both of its loads).
  auto page_blk = [&](int pg) -> int64_t {
    if constexpr (PG)
      return min(max((int64_t)kconst(a.table + (int64_t)b * a.max_pages + pg)[0], (int64_t)0),
                 a.n_blocks - 1);
    else
      return 0;
  };
  auto page_rsrc = [&](const uint8_t* pool, int64_t bytes, rsrc_t whole, int pg, int64_t blk,
                       bool valid, uint32_t& so) -> rsrc_t {
    so = 0u;
    if (!valid) return nul;
    if constexpr (PG) {
      return buf_rsrc(pool + (blk * a.H_kv + h) * bytes, bytes);
    } else {
      so = (uint32_t)((int64_t)pg * a.H_kv * bytes);
      return whole;
    }
  };
  auto load_k = [&](int pgk, int64_t blk, bool valid) {
    uint32_t so;
    const rsrc_t krs_p = page_rsrc(a.k_pages, a.kpb, krs, pgk, blk, valid, so);
    const rsrc_t krs = krs_p;
#pragma unroll
    for (int ks = 0; ks < KL; ++ks) {
      const int c0 = 64 * ks + 16 * qb;
      wL[ks] = c0 < D ? bload16(krs, oct * D + c0, so) : v4u{0, 0, 0, 0};
    }
#pragma unroll
    for (int ks = 0; ks < KHM; ++ks) {
      // ranks past n_sal read other bytes of the page: their A columns are zero
      const uint32_t h0 = kN * D / 8 + 64 * ks + 16 * qb + (2 * oct) * n_sal;
      hr0[ks] = bload20(krs, h0, so);
      hr1[ks] = bload20(krs, h0 + n_sal, so);
    }
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      sv[kg] = bload8(krs, sOff + 2 * (kg * D + 4 * (lane % JL)), so);
      zv[kg] = bload8(krs, zOff + 2 * (kg * D + 4 * (lane % JL)), so);
    }
  };
  // Value side of one page: the scales and offsets of keys 8 oct + b in the value group of
  // block qb (the lanes of row bk hold block bk's; the other rows fetch them across lanes when
  // the block's digits are formed); code bytes of this lane's p.V tile columns per K-step.
  const uint32_t vS = kN * D / 4 + 2 * 8 * oct;  // S [NGV][N] fp16 after the codes, then Z
  // value groups are 32 << vg_shift channels: block bk belongs to group bk >> vg_shift and
  // starts one where (bk & vg_mask) == 0
  const int vg_shift = __builtin_ctz((uint32_t)a.g_V) - 5;
  const int vg_mask = (1 << vg_shift) - 1;
  const int gq = min(qb, NBLK - 1) >> vg_shift;
  v4u sSo, zZo;
  v4u cv[NBLK][2];
  auto load_v = [&](int pgv, int64_t blk, bool valid) {
    uint32_t vso;
    const rsrc_t vrs_p = page_rsrc(a.v_pages, a.vpb, vrs, pgv, blk, valid, vso);
    const rsrc_t vrs = vrs_p;
    sSo = bload16(vrs, vS + 2 * gq * kN, vso);
    zZo = bload16(vrs, vS + 2 * (NGV + gq) * kN, vso);
#pragma unroll
    for (int bk = 0; bk < NBLK; ++bk)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        cv[bk][ks] = bload16(vrs, (8 * bk + vcol) * kN + 64 * ks + 16 * qb, vso);
  };
  // Pages of this split: split, split + page_splits, ...  (a split past the last page drops
  // the loads of its first one)
  const int step = a.page_splits, p0 = split;
  int64_t blk_cur = page_blk(p0);  // p0 < page_splits <= max_pages: inside the table row
  load_k(p0, blk_cur, true);
  if constexpr (!kLate) load_v(p0, blk_cur, true);

  const auto mrow = kconst(a.mask + bh * a.words);
  const uint32_t mw0 = mrow[0], mw1 = a.words > 1 ? mrow[1] : 0u;
  const int n_pages = min(max(kconst(&a.lens[b].n_pages)[0], 0), a.max_pages);
  // A split past the last page runs its set-up and no page: its partial is m = -inf, l = 0,
  // o = 0.  (No early exit: a branch that stores its partial early would force waits for all
  // loads in flight at the point where it rejoins.)

  // LDS: q.K digit table T [KG][NT][16][TL] bytes; p.V digit table W [NT][16][kWS] bytes (one
  // value group at a time);
  // bias [KG][NH][2] f32 (a head's sums over its two 16-lane rows); scaled queries [NH][D] f32.
  uint8_t* T = lds;
  uint8_t* W = lds + a.lds_T;
  float* biasl = reinterpret_cast<float*>(W + NT * 16 * kWS);
  float* qs = biasl + 2 * 4 * NH;

  // ---- once per split: clear the digit table, salient ranks, scaled queries
  for (int i = lane * 16; i < a.lds_T; i += 64 * 16) *reinterpret_cast<v4u*>(T + i) = v4u{0, 0, 0, 0};
  // Upper-bit digit rows: the digits of a salient channel are the same words as its LSB digits
  // (same qt S product), placed at the channel's salient rank.  Each LSB prep unit scatters the
  // digit bytes of its salient channels there; hoff[k] holds, for the unit's 4 channels, the
  // byte offset (within one key group's table) of digit row 0 at that rank, two to a word, or
  // a padding column of rows 0..3 (never read by the A loads) for a channel that is not salient.
  uint32_t hoff[UK][2];
#pragma unroll
  for (int k = 0; k < UK; ++k) {
    const int u = lane + 64 * k;
    const int hu = u / JL, j = u % JL;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = u < NT * D ? salient_rank2(mw0, mw1, 4 * j + i, D, a.pairing, a.n_hi) : -1;
      o[i] = r >= 0 ? (uint32_t)(((hu / 4) * 16 + 4 * (hu % 4)) * TL + 64 * KL + r)
                    : (uint32_t)(64 * (KL + KHM));
    }
    hoff[k][0] = o[0] | (o[1] << 16);
    hoff[k][1] = o[2] | (o[3] << 16);
  }
  // scaled queries go to LDS (qs) and are read back per page; the registers keep only their
  // largest magnitude over the group's heads
  float qmax = 0.0f;
#pragma unroll
  for (int k = 0; k < UK; ++k) {
    const int u = lane + 64 * k;
    const v4f q4 = v4f{f16lo(qq[k].x), f16hi(qq[k].x), f16lo(qq[k].y), f16hi(qq[k].y)} * a.qscale;
    qmax = fmaxf(qmax, fmaxf(fmaxf(fabsf(q4[0]), fabsf(q4[1])), fmaxf(fabsf(q4[2]), fabsf(q4[3]))));
    if (u < NT * D) *reinterpret_cast<v4f*>(qs + 4 * u) = q4;
  }
  qmax = wave_max_nonneg(qmax);

  // running softmax state of head 4t + lane/16; p.V accumulators per 16-channel tile (C
  // layout: column lane % 16), value-offset sums per value group (kept at the group's first
  // block of 32 channels; the other blocks' entries stay zero)
  float m_run[NT], l_run[NT];
  float zacc[NT][NBLK];
  float acc[NT][NTV];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.0f;
#pragma unroll
    for (int bk = 0; bk < NBLK; ++bk) zacc[t][bk] = 0.0f;
#pragma unroll
    for (int v = 0; v < NTV; ++v) acc[t][v] = 0.0f;
  }

  for (int pg = p0; pg < n_pages; pg += step) {
    const bool more = pg + step < n_pages;
    const int64_t blk_next = page_blk(more ? pg + step : pg);

    // ---- key scales: page maximum -> per-head fixed-point exponent
    uint32_t smax = 0u;
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
      smax = pk_max_u16(smax, pk_max_u16(sv[kg].x, sv[kg].y));
    }
    smax = wave_max_u32(max(smax & 0xFFFFu, smax >> 16));
    const float Smax = (float)__builtin_bit_cast(_Float16, (uint16_t)smax);
    // 2^sigma with |qt S 2^sigma| < 2^30 for every channel of every head of the group (one
    // fixed point for the page: a head with smaller queries keeps fewer of the 30 bits, its
    // logits the same absolute resolution 2^-sigma per term)
    int sigma = 0;
    {
      const float M = qmax * Smax;
      const int e = (int)((__builtin_bit_cast(uint32_t, M) >> 23) & 0xFF) - 127;
      if (M > 0.0f) sigma = min(max(29 - e, -126), 126);
    }
    const float sc = pow2i(sigma), inv2s = pow2i(-sigma);

    // ---- digit table, LSB part, and the Z bias of each head
#pragma unroll
    for (int k = 0; k < UK; ++k) {
      const int u = lane + 64 * k;
      const int hu = u / JL, j = u % JL;
      const bool ok = u < NT * D;
      const v4f qv = ok ? *reinterpret_cast<const v4f*>(qs + 4 * u) : v4f{0.0f, 0.0f, 0.0f, 0.0f};
      const v4f qsc = qv * sc;  // exact: a power of two
#pragma unroll
      for (int kg = 0; kg < KG; ++kg) {
        // qt 2^sigma S rounded once (fp16 S widened exactly inside the mixed-precision fma)
        const float m4[4] = {fma_mix_lo(qsc[0], sv[kg].x, 0.0f), fma_mix_hi(qsc[1], sv[kg].x, 0.0f),
                             fma_mix_lo(qsc[2], sv[kg].y, 0.0f), fma_mix_hi(qsc[3], sv[kg].y, 0.0f)};
        uint32_t y[4], dg[4];
        float bz = 0.0f;
        bz = fma_mix_lo(qv[0], zv[kg].x, bz);
        bz = fma_mix_hi(qv[1], zv[kg].x, bz);
        bz = fma_mix_lo(qv[2], zv[kg].y, bz);
        bz = fma_mix_hi(qv[3], zv[kg].y, bz);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = digits4((int)m4[i]);
        transpose4(y, dg);
        // sums over the unit's lanes of one head within a 16-lane row (DPP only); a head
        // spanning two rows leaves its two row sums in LDS and the reader adds them
        bz = group_sum<(JL < 16 ? JL : 16)>(bz);
        if (ok) {
          const int t = hu / 4, hl = hu % 4;
          uint8_t* row = T + ((kg * NT + t) * 16 + 4 * hl) * TL + 4 * j;
#pragma unroll
          for (int d = 0; d < 4; ++d) *reinterpret_cast<uint32_t*>(row + d * TL) = dg[d];
          if (j % (JL < 16 ? JL : 16) == 0) biasl[2 * (kg * NH + hu) + (j >> 4)] = bz;
        }
        // the same digit words at the salient ranks of the upper-bit rows
        uint8_t* tb = T + kg * NT * 16 * TL;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint8_t* p = tb + ((hoff[k][i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
          p[0] = (uint8_t)y[i];
          p[TL] = (uint8_t)(y[i] >> 8);
          p[2 * TL] = (uint8_t)(y[i] >> 16);
          p[3 * TL] = (uint8_t)(y[i] >> 24);
        }
      }
    }
    wave_sync();  // the LSB and upper-bit digits are in LDS

    // ---- A operands (digit rows) of every tile and key group
    v4i A[KG][NT][KL + KHM];
#pragma unroll
    for (int kg = 0; kg < KG; ++kg) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int ks = 0; ks < KL + KHM; ++ks)
          A[kg][t][ks] = *reinterpret_cast<const v4i*>(T + ((kg * NT + t) * 16 + (lane & 15)) * TL +
                                                       64 * ks + 16 * qb);
    }
    float bias[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float* bp = biasl + 2 * (kg_lane * NH + 4 * t + qb);
      bias[t] = JL > 16 ? bp[0] + bp[1] : bp[0];
    }

    // ---- q.K: tile b holds keys 8 oct + b; the lane's q.K output head is 4t + qb
    v4u wH0[KHM], wH1[KHM];
#pragma unroll
    for (int ks = 0; ks < KHM; ++ks) {
      const uint32_t h0 = 64 * ks + 16 * qb + (2 * oct) * n_sal;  // alignment as loaded
      wH0[ks] = align20(hr0[ks], h0);
      wH1[ks] = align20(hr1[ks], h0 + n_sal);
    }
    float lg[NT][8];
#define PNMIX_QK_TILE(BB)                                                                      \
    {                                                                                          \
      v4i bL[KL], bH[KHM];                                                                     \
      _Pragma("unroll") for (int ks = 0; ks < KL; ++ks) {                                      \
        v4u w = wL[ks];                                                                        \
        bL[ks] = v4i{(int)lsb_field<BB>(w[0]), (int)lsb_field<BB>(w[1]),                       \
                     (int)lsb_field<BB>(w[2]), (int)lsb_field<BB>(w[3])};                      \
      }                                                                                        \
      _Pragma("unroll") for (int ks = 0; ks < KHM; ++ks) {                                     \
        v4u w = (BB < 4) ? wH0[ks] : wH1[ks];                                                  \
        bH[ks] = v4i{(int)hi_field<BB>(w[0]), (int)hi_field<BB>(w[1]),                         \
                     (int)hi_field<BB>(w[2]), (int)hi_field<BB>(w[3])};                        \
      }                                                                                        \
      _Pragma("unroll") for (int t = 0; t < NT; ++t) {                                         \
        v4i csel = v4i{0, 0, 0, 0};                                                            \
        _Pragma("unroll") for (int kg = 0; kg < KG; ++kg) {                                    \
          v4i c = v4i{0, 0, 0, 0};                                                             \
          _Pragma("unroll") for (int ks = 0; ks < KL; ++ks)                                    \
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[kg][t][ks], bL[ks], c, 0, 0, 0);       \
          _Pragma("unroll") for (int ks = 0; ks < KHM; ++ks)                                   \
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[kg][t][KL + ks], bH[ks], c, 0, 0, 0);    \
          csel = (KG == 1 || kg == kg_lane) ? c : csel;                                        \
        }                                                                                      \
        lg[t][BB] = __builtin_fmaf(combine4(csel), inv2s * kInvSL[BB], bias[t]);               \
      }                                                                                        \
    }
    PNMIX_QK_TILE(0) PNMIX_QK_TILE(1) PNMIX_QK_TILE(2) PNMIX_QK_TILE(3)
    PNMIX_QK_TILE(4) PNMIX_QK_TILE(5) PNMIX_QK_TILE(6) PNMIX_QK_TILE(7)
#undef PNMIX_QK_TILE

    // ---- the key side of this page is consumed: fetch the next page's (with several head
    // tiles: fetch the value side now and the next keys after p.V, to keep fewer registers live)
    if constexpr (kLate) {
      load_v(pg, blk_cur, true);
    } else {
      load_k(pg + step, blk_next, more);
    }

    // ---- p.V fixed point, per head: x = rne(p S 2^sh) with 2^sh above the head's largest
    // p on this page times the page's largest value scale, so 0 <= x <= 2^22 (22 bits relative
    // to the page's own largest term, whatever the running maximum of earlier pages).  The
    // bound has headroom: top is a rounded product and p 2^sh and x round once more each, so x
    // can reach 2^22 (and a few units more); the top digit of x + 0x8080 then stays at most 65,
    // far below the int8 sign bit.
    uint32_t svm2 = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) svm2 = pk_max_u16(svm2, sSo[e]);  // S >= 0: bit order
    const float svmax = wave_max_nonneg(fmaxf(f16lo(svm2), f16hi(svm2)));

    // ---- online softmax of every head tile: pw = p 2^sh (the p.V fixed-point scale of the
    // head), the running maximum, sum and rescaled accumulators
    float pw[NT][8], inv_sv[NT], pscl[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float pm = lg[t][0];
#pragma unroll
      for (int bb = 1; bb < 8; ++bb) pm = fmaxf(pm, lg[t][bb]);
      pm = row_max16(pm);
      const float mn = fmaxf(m_run[t], pm);
      const float alpha = __builtin_amdgcn_exp2f(m_run[t] - mn);
      m_run[t] = mn;
      int sh;
      {
        const float top = __builtin_amdgcn_exp2f(pm - mn) * svmax;  // >= every w of this head
        int e = 0;
        if (top > 0.0f) e = (int)((__builtin_bit_cast(uint32_t, top) >> 23) & 0xFF) - 127;
        sh = min(max(21 - e, -126), 126);
      }
      inv_sv[t] = pow2i(-sh);
      pscl[t] = inv_sv[t] * vfw;
      // p 2^sh = 2^(lg - (mn - sh)) in one exp2; the sum of p is that of p 2^sh times 2^-sh
      const float msh = mn - (float)sh;
      float ps = 0.0f;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        pw[t][bb] = __builtin_amdgcn_exp2f(lg[t][bb] - msh);
        ps += pw[t][bb];
      }
      l_run[t] = __builtin_fmaf(ps, inv_sv[t], l_run[t] * alpha);
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int v = 0; v < NTV; ++v) acc[t][v] *= alpha;
#pragma unroll
        for (int bk = 0; bk < NBLK; ++bk) zacc[t][bk] *= alpha;
      }
    }

    // ---- p.V per block of 32 channels (one value group, or part of one): where a group
    // starts, the digits of w = p S of every head tile go to the digit table W and the group's
    // offset term sum_t p Z is accumulated on the vector ALU; then tile v = (bk, field pair f)
    // of every head tile: column n is channel 4 (8 bk + n % 8) + f + 2 (n / 8); rows (head,
    // digit); K = 64 keys.  The masked value codes (B operand) are formed once per tile and
    // serve every head tile.
#pragma unroll
    for (int bk = 0; bk < NBLK; ++bk) {
      if (bk == 0 || (bk & vg_mask) == 0) {
        // block bk's scales and offsets from the lanes of row bk (same octet)
        v4u ss, zz;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int src = 4 * ((lane & 15) + 16 * bk);
          ss[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)sSo[e]);
          zz[e] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)zZo[e]);
        }
        if (bk) wave_sync();  // the previous group's rows of W are read
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float zs = 0.0f;
          uint32_t x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            zs = fma_mix_lo(pw[t][2 * e], zz[e], zs);
            zs = fma_mix_hi(pw[t][2 * e + 1], zz[e], zs);
            // x + 0x8080 in the float's bits 0..22 (byte 2 <= 65)
            x[2 * e] = __builtin_bit_cast(uint32_t, fma_mix_lo(pw[t][2 * e], ss[e], kTwo23b));
            x[2 * e + 1] = __builtin_bit_cast(uint32_t, fma_mix_hi(pw[t][2 * e + 1], ss[e], kTwo23b));
          }
          zacc[t][bk] = __builtin_fmaf(zs, inv_sv[t], zacc[t][bk]);
          uint32_t d0[3], d1[3];
          transpose3(x, d0);
          transpose3(x + 4, d1);
          // digit rows 0, 1: the balanced digits (bytes xor 0x80); row 2: the top digit
          uint8_t* row = W + (t * 16 + 4 * qb) * kWS + 8 * oct;
          *reinterpret_cast<uint2*>(row) = make_uint2(d0[0] ^ 0x80808080u, d1[0] ^ 0x80808080u);
          *reinterpret_cast<uint2*>(row + kWS) = make_uint2(d0[1] ^ 0x80808080u, d1[1] ^ 0x80808080u);
          *reinterpret_cast<uint2*>(row + 2 * kWS) = make_uint2(d0[2], d1[2]);
        }
        wave_sync();  // the w digits of this group are in LDS
      }
      v4i A0[NT], A1[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint8_t* wrow = W + (t * 16 + (lane & 15)) * kWS + 16 * qb;
        A0[t] = *reinterpret_cast<const v4i*>(wrow);
        A1[t] = *reinterpret_cast<const v4i*>(wrow + 64);
      }
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int v = 2 * bk + f;
        v4i Bv[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const v4u w = cv[bk][ks];
#pragma unroll
          for (int e = 0; e < 4; ++e) Bv[ks][e] = (int)((f == 0 ? w[e] : (w[e] >> 2)) & vmask);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          v4i c = v4i{0, 0, 0, 0};
          c = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0[t], Bv[0], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1[t], Bv[1], c, 0, 0, 0);
          acc[t][v] = __builtin_fmaf(combine_pv(c), pscl[t], acc[t][v]);
        }
      }
    }
    if constexpr (kLate) {
      load_k(pg + step, blk_next, more);
    } else {
      load_v(pg + step, blk_next, more);
    }
    blk_cur = blk_next;
    wave_sync();  // T, W and Sl are rewritten by the next page (and by the partial)
  }

  // ---- partials of this split: head 4t + qb, channel of tile v for column lane % 16
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float lt = row_sum16(l_run[t]);
    // the offset sum of each block's value group (held by the group's first block)
    float zs[NBLK];
#pragma unroll
    for (int bk = 0; bk < NBLK; ++bk) {
      zs[bk] = row_sum16(zacc[t][bk]);
      if (bk > 0 && (bk & vg_mask) != 0) zs[bk] = zs[bk - 1];
    }
    const int hh = 4 * t + qb;
    if (hh < ng) {
#pragma unroll
      for (int v = 0; v < NTV; ++v) {
        const int c = 4 * (8 * (v / 2) + (lane & 7)) + (v % 2) + 2 * ((lane >> 3) & 1);
        po.o(hh * D + c, acc[t][v] + zs[v / 2]);
      }
      if ((lane & 15) == 0) {
        po.ml(hh, m_run[t], lt);
      }
    }
  }
}

// ----------------------------------------------------------------------------------- merge

// Second launch: one workgroup of 256 per (sequence, query head).  out = sum_s 2^(m_s - m) o_s /
// sum_s 2^(m_s - m) l_s with m = max_s m_s (log2 units).  Thread (split lane sl, channel quad cq)
// loads (m, l, o) of its splits sl, sl + SL, ... CH at a time (CH = the number of splits a lane
// has, rounded up to a power of two, at most kMergeChunk: a lane issues no loads for splits
// that do not exist beyond that rounding) and folds them in ascending order with the online rule (m, l, o) <- (m', l 2^(m - m') +
// l_s 2^(m_s - m'), same for o), m' = max(m, m_s); the SL lane results are folded the same way,
// in ascending sl, through LDS.  A sequence with no tokens (every m_s = -inf) gets out = 0.
constexpr int kMergeChunk = 8;
struct MergeAcc {
  float m, l;
  v4f o;
  __device__ __forceinline__ void fold(float ms, float ls, const v4f& os) {
    if (ms == -INFINITY) return;  // an empty split
    const float mn = fmaxf(m, ms);
    const float a = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    const float w = __builtin_amdgcn_exp2f(ms - mn);
    l = __builtin_fmaf(w, ls, l * a);
    o = o * a + w * os;
    m = mn;
  }
};
template <int D, int CH>
__global__ void __launch_bounds__(256) decode_merge_kernel(DecodeArgs a) {
  constexpr int Q = D / 4, SL = 256 / Q;
  __shared__ v4f red_o[256];
  __shared__ float red_m[256], red_l[256];
  const int tid = threadIdx.x;
  const int bhq = blockIdx.x;  // b * H_q + hq
  const int b = bhq / a.H_q, hq = bhq % a.H_q;
  const int ng = a.n_g, S = a.splits;
  const int h = hq / ng, hh = hq % ng;
  const int64_t bh = (int64_t)b * a.H_kv + h;
  const int cq = tid % Q, sl = tid / Q;
  // partial r = (split s, head hh) of this (sequence, KV head); loads past the last split read
  // zero (buffer bounds) and are not folded
  const rsrc_t mlr = buf_rsrc(a.part_ml + bh * S * ng * 2, (int64_t)S * ng * 2 * 4);
  const rsrc_t por = buf_rsrc(a.part_o + bh * S * ng * D, (int64_t)S * ng * D * 4);
  MergeAcc acc{-INFINITY, 0.0f, v4f{0.0f, 0.0f, 0.0f, 0.0f}};
  for (int s0 = sl; s0 < S; s0 += CH * SL) {
    v4u ob[CH];
    uint32_t mb[CH], lb[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int r = (s0 + j * SL) * ng + hh;
      ob[j] = bload16(por, (uint32_t)(4 * (r * D + 4 * cq)), 0u);
      mb[j] = __builtin_amdgcn_raw_buffer_load_b32(mlr, (uint32_t)(8 * r), 0u, 0);
      lb[j] = __builtin_amdgcn_raw_buffer_load_b32(mlr, (uint32_t)(8 * r + 4), 0u, 0);
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (s0 + j * SL < S)
        acc.fold(__builtin_bit_cast(float, mb[j]), __builtin_bit_cast(float, lb[j]),
                 __builtin_bit_cast(v4f, ob[j]));
  }
  red_o[tid] = acc.o;
  red_m[tid] = acc.m;
  red_l[tid] = acc.l;
  __syncthreads();
  if (tid < Q) {
#pragma unroll 4
    for (int g = 1; g < SL; ++g) acc.fold(red_m[g * Q + tid], red_l[g * Q + tid], red_o[g * Q + tid]);
    const float inv = acc.l > 0.0f ? 1.0f / acc.l : 0.0f;
    *reinterpret_cast<v4f*>(a.out + (int64_t)bhq * D + 4 * tid) = acc.o * inv;
  }
  // Fused append: every split of this call has read the cache and the lengths, so the new rows
  // go in now, one (sequence, KV head) per block of its first query head, and the advanced
  // lengths into lens_out.
  if (a.k_new && hh == 0) {
    const pnmix_seq_len L = a.lens[b];
    int kind, row;
    append_slot(L, a.N_s, kind, row);
    if (kind != 2 && tid < 2 * (D / 8)) {
      const bool isv = tid >= D / 8;
      const int c8 = isv ? tid - D / 8 : tid;
      const int cap = kind == 0 ? a.N_s : kN;
      uint16_t* dst = const_cast<uint16_t*>(kind == 0 ? (isv ? a.v_sink : a.k_sink)
                                                      : (isv ? a.v_res : a.k_res));
      const uint16_t* src = (isv ? a.v_new : a.k_new) + bh * D + 8 * c8;
      *reinterpret_cast<v4u*>(dst + (bh * cap + row) * D + 8 * c8) =
          *reinterpret_cast<const v4u*>(src);
    }
    if (h == 0 && tid == 0) {
      pnmix_seq_len Lo = L;
      if (kind == 0) Lo.sink_len = row + 1;
      if (kind == 1) Lo.res_len = row + 1;
      a.lens_out[b] = Lo;
    }
  }
}

// Waves per workgroup the split kernel is compiled for: eight for the instantiations that run
// two waves per SIMD, four (one per SIMD) otherwise.
template <int D, int NT, int KG, int KH>
struct KernelWaves {
  static constexpr bool two = (NT == 1 && KG <= 2) || (NT == 2 && KG == 1 && (D <= 64 || KH == 1));
  static constexpr int max_nw = two ? 8 : 4;
};

// One launch per decode call.  Wave w of workgroup x takes split x nw + w of its (sequence, KV
// head): the first page_splits walk packed pages, the next ones take one 64-token chunk each of
// the fp16 sink and residual rows (32-token pieces strided over them), any further ones are
// empty.  With fold16 (one wave per workgroup) the fp16 pieces have no waves of their own: the
// page splits take them after their pages, the last split first.  With one wave per workgroup
// the split writes its partial to the workspace; with nw > 1 the waves leave their partials in
// their LDS slices and the workgroup merges them into one partial (same log-sum-exp rule as
// the merge kernel), so the merge kernel reads nw times fewer.
// Two waves per SIMD (at most 256 registers) where the compiler fits them without spills:
// one head tile with at most two key groups, or two head tiles with one key group (and one
// upper-bit K-step at d = 128).
template <int D, int NT, int KG, int KH, bool PG>
__global__ void __launch_bounds__((64 * KernelWaves<D, NT, KG, KH>::max_nw))
__attribute__((amdgpu_waves_per_eu((KernelWaves<D, NT, KG, KH>::two ? 2 : 1))))
decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int nw = a.nw;
  const int wv = nw > 1 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  const int split = (int)blockIdx.x * nw + wv;
  const int64_t bh = blockIdx.y;
  const int ng = a.n_g;
  uint8_t* wl = lds + (size_t)wv * a.lds_wave;
  const int64_t pbase = (bh * a.splits + split) * ng;  // nw == 1
  lds_f32* const st = (lds_f32*)(wl);
  const PartOut po{a.part_o + pbase * D, a.part_ml + pbase * 2, st, st + ng * D, nw > 1};
  // One call site of each region (the page split, then the fp16 rows).  The fp16 pieces go to
  // splits of their own (split - page_splits of n16, pieces strided by n16), or with fold16 to
  // the page splits, last split first (piece i to split page_splits - 1 - i, strided by
  // page_splits); such a wave leaves its page partial in LDS past the V^T staging and the fp16
  // pass merges it into the one partial it stores.
  const bool pages = split < a.page_splits;
  int first16 = -1, stride16 = 1;
  if (a.fold16 > 0) {
    if (pages && a.page_splits - 1 - split < a.fold16) {
      first16 = a.page_splits - 1 - split;
      stride16 = a.page_splits;
    }
  } else if (!pages && split < a.page_splits + a.n16) {
    first16 = split - a.page_splits;
    stride16 = a.n16;
  }
  lds_f32* const pl = (lds_f32*)(wl + kVtBytes<D>);
  const bool merge = pages && first16 >= 0;
  if (pages) page_split<D, NT, KG, KH, PG>(a, wl, split, bh, merge ? PartOut{po.go, po.gml, pl, pl + ng * D, true} : po);
  if (first16 >= 0) {
    fp16_split<D>(a, bh, po, first16, stride16, wl, merge ? pl : nullptr);
  } else if (!pages) {
    write_empty_partial<D>(a, po);
  }
  if (nw == 1) return;
  __syncthreads();  // every wave's partial is in its LDS slice
  const int64_t pb = (bh * a.splits + blockIdx.x) * ng;
  const int nthr = 64 * nw;
  for (int i = threadIdx.x; i < ng * (D + 1); i += nthr) {
    const int hh = i < ng * D ? i / D : i - ng * D;
    float M = -INFINITY;
    for (int w = 0; w < nw; ++w)
      M = fmaxf(M, reinterpret_cast<const float*>(lds + (size_t)w * a.lds_wave)[ng * D + 2 * hh]);
    float r = 0.0f;
    for (int w = 0; w < nw; ++w) {
      const float* st = reinterpret_cast<const float*>(lds + (size_t)w * a.lds_wave);
      const float mw = st[ng * D + 2 * hh];
      const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      r = __builtin_fmaf(f, i < ng * D ? st[i] : st[ng * D + 2 * hh + 1], r);
    }
    if (i < ng * D) {
      a.part_o[pb * D + i] = r;
    } else {
      a.part_ml[(pb + hh) * 2 + 0] = M;
      a.part_ml[(pb + hh) * 2 + 1] = r;
    }
  }
}

// ---------------------------------------------------------------------------------- host

// 4-head tiles of the GQA group; 3 tiles run as 4 (the extra heads are zero)
static int n_tiles(const pnmix_cfg& c) {
  const int t = (c.H_q / c.H_kv + 3) / 4;
  return t == 3 ? 4 : t;
}

// 64-rank K-steps over the upper-bit plane: two only for d = 128 with more than 64 salient
// channels
static int hi_steps(const pnmix_cfg& c) { return (c.d == 128 && 2 * c.n_hi_pairs > 64) ? 2 : 1; }

static size_t lds_T_bytes(const pnmix_cfg& c) {
  const int KL = (c.d + 63) / 64;
  const int TL = 64 * (KL + hi_steps(c)) + 16;
  return (size_t)(c.N / c.G) * n_tiles(c) * 16 * TL;
}

static size_t lds_bytes(const pnmix_cfg& c) {
  const int NT = n_tiles(c);
  const size_t W = (size_t)NT * 16 * kWS;  // one value group's rows of every head tile
  return lds_T_bytes(c) + W + 2 * 4 * 4 * NT * 4 + (size_t)4 * NT * c.d * 4;
}

static size_t lds_fp16_bytes(const pnmix_cfg& c) {
  return (size_t)c.d * 36 * 2;  // V^T [d][32 tokens + 4] halves (kVtBytes)
}

// LDS slice of one wave: the larger of the page and fp16 layouts, and at least the partial the
// wave leaves there for its workgroup's merge
static size_t lds_wave_bytes(const pnmix_cfg& c) {
  const size_t ng = (size_t)(c.H_q / c.H_kv);
  const size_t b = std::max(std::max(lds_bytes(c), lds_fp16_bytes(c)), ng * (c.d + 2) * 4);
  return (b + 15) & ~(size_t)15;
}

// f.template run<D, NT, KG, KH>() for the split kernel instantiation of the configuration
template <int D, int NT, int KG, class F>
static auto dispatch_kh(const pnmix_cfg& c, const F& f) {
  if constexpr (D == 128) {
    if (hi_steps(c) == 2) return f.template run<D, NT, KG, 2>();
  }
  return f.template run<D, NT, KG, 1>();
}
template <int D, int NT, class F>
static auto dispatch_kg(const pnmix_cfg& c, const F& f) {
  switch (c.N / c.G) {
    case 1: return dispatch_kh<D, NT, 1>(c, f);
    case 2: return dispatch_kh<D, NT, 2>(c, f);
    default: return dispatch_kh<D, NT, 4>(c, f);
  }
}
template <int D, class F>
static auto dispatch_nt(const pnmix_cfg& c, const F& f) {
  switch (n_tiles(c)) {
    case 1: return dispatch_kg<D, 1>(c, f);
    case 2: return dispatch_kg<D, 2>(c, f);
    default: return dispatch_kg<D, 4>(c, f);
  }
}
template <class F>
static auto dispatch(const pnmix_cfg& c, const F& f) {
  switch (c.d) {
    case 32: return dispatch_nt<32>(c, f);
    case 64: return dispatch_nt<64>(c, f);
    default: return dispatch_nt<128>(c, f);
  }
}

// Device limits (defaults without a device): compute units, dynamic LDS per workgroup.
static const hipDeviceProp_t* device_prop() {
  static hipDeviceProp_t prop;
  static const bool ok = [] {
    int dev = 0;
    return hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess;
  }();
  return ok ? &prop : nullptr;
}
static int device_cus() {
  const hipDeviceProp_t* p = device_prop();
  return p && p->multiProcessorCount > 0 ? p->multiProcessorCount : 256;
}
static size_t device_lds_per_block() {
  const hipDeviceProp_t* p = device_prop();
  return p && p->sharedMemPerBlock > 0 ? p->sharedMemPerBlock : 65536;
}

struct MaxWaves {
  template <int D, int NT, int KG, int KH>
  int run() const {
    return KernelWaves<D, NT, KG, KH>::max_nw;
  }
};

// dynamic LDS above 64 KiB has to be allowed per kernel
template <int D, int NT, int KG, int KH, bool PG>
static hipError_t allow_lds(size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<D, NT, KG, KH, PG>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Workgroups of the split kernel resident per compute unit (the runtime's occupancy for this
// instantiation, block size and LDS size).
struct BlocksPerCu {
  size_t lds;
  int threads;
  template <int D, int NT, int KG, int KH>
  int run() const {
    int n = 0;
    if (allow_lds<D, NT, KG, KH, false>(lds) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_kernel<D, NT, KG, KH, false>, threads,
                                                     lds) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      return std::max(1, 8 / (threads / 64));
    }
    return n;
  }
};

// Split plan.  Large batches (>= 128 (sequence, KV head) items): one wave per workgroup, and the
// fp16 rows either in one split of their own or spread over the page splits in 32-token pieces,
// the last split (which has the fewest pages) first.  Small batches: workgroups of nw waves (as many as
// the instantiation and the LDS allow) merge their waves' partials on chip, and the number of
// fp16 splits is searched too.  Cost = rounds of resident workgroups x (pages per split + 1 for
// the set-up), the fp16 splits' chunks counting half a page each; ties go to more page splits.
// At most kMergeSplits partials per (sequence, KV head) (the merge reads every one).
// The matrix-core split kernel serves (b_H, b_L, b_V) = (3, 1, 2) with value groups of at least
// 32 channels (a p.V tile spans 32 channels of one group); every other setting takes the
// generic kernel of decode_generic.hip.
bool decode_fast_path(const pnmix_cfg& c) {
  return c.b_H == 3 && c.b_L == 1 && c.b_V == 2 && c.g_V >= 32;
}

// Generic kernel plan: one 256-thread workgroup per (sequence, KV head, split) walking chunks
// of 128 tokens (sinks, pages, residual).  Cost = rounds of resident workgroups x (chunks per
// split + 1 for the set-up), ties to more splits; at most one split per chunk and kMergeSplits
// in all.  (Whole rounds matter: with three workgroups per CU, Qwen3-8B at B = 32 (256 items,
// 65 chunks) runs 116 us at 3 splits (one round) and 152 us at 4 (two, the second a third
// full).)
static DecodePlan generic_plan(const pnmix_cfg& c, int B, int max_pages) {
  DecodePlan p;
  const long long items = std::max<long long>((long long)B * c.H_kv, 1);
  const int chunks = max_pages + 2;
  p.lds_wave = generic_lds_bytes(c);
  p.lds_bytes = p.lds_wave;
  const long long resident = (long long)generic_blocks_per_cu(c, p.lds_bytes) * device_cus();
  int best_s = 1;
  long long best = -1;
  for (int s = 1; s <= std::min(chunks, kMergeSplits); ++s) {
    const long long rounds = (items * s + resident - 1) / resident;
    const long long cost = rounds * ((chunks + s - 1) / s + 1);
    if (best < 0 || cost <= best) {
      best = cost;
      best_s = s;
    }
  }
  p.splits = best_s;
  p.page_splits = p.splits;
  p.n16 = 0;
  p.fold16 = 0;
  p.nw = 1;
  p.pages_per_split = (max_pages + p.splits - 1) / p.splits;
  const int ng = c.H_q / c.H_kv;
  const size_t per = (size_t)items * p.splits * ng;
  const size_t o_bytes = (per * c.d * sizeof(float) + 255) & ~(size_t)255;
  p.ws_bytes = o_bytes + ((per * 2 * sizeof(float) + 255) & ~(size_t)255);
  return p;
}

DecodePlan decode_plan(const pnmix_cfg& c, int B, int max_pages) {
  if (!decode_fast_path(c)) return generic_plan(c, B, max_pages);
  DecodePlan p;
  const long long items = std::max<long long>((long long)B * c.H_kv, 1);
  p.lds_wave = lds_wave_bytes(c);
  const int chunks = (c.N_s + c.N + 63) / 64;
  int nw = 1;
  if (items < 128) {
    nw = dispatch(c, MaxWaves{});
    while (nw > 1 && (size_t)nw * p.lds_wave > device_lds_per_block()) nw /= 2;
  }
  p.nw = nw;
  p.lds_bytes = (size_t)nw * p.lds_wave;
  const int bpc = dispatch(c, BlocksPerCu{p.lds_bytes, 64 * nw});
  const long long resident = (long long)bpc * device_cus();  // workgroups
  // Costs in quarter pages: a page 4, a wave's set-up 4, a 64-token chunk of a split of its own
  // 2, a 32-token piece on a page wave kPieceCost.
  const int pieces = (c.N_s + c.N + 31) / 32;
  const size_t ng = (size_t)(c.H_q / c.H_kv);
  // with the pieces spread, a wave's page partial waits in LDS past the V^T staging
  const size_t fold_wave = std::max(p.lds_wave, (lds_fp16_bytes(c) + ng * (c.d + 2) * 4 + 15) & ~(size_t)15);
  int ps = 0, n16 = nw == 1 ? (items >= 128 ? 1 : chunks) : 1, fold = 0;
  if (max_pages > 0) {
    long long best = -1;
    const int n16_lo = n16, n16_hi = nw == 1 ? n16 : chunks;
    for (int f = n16_lo; f <= n16_hi; ++f) {
      const int f16 = nw == 1 ? 0 : 2 * ((chunks + f - 1) / f);
      const int ps_max = std::min(max_pages, kMergeSplits * nw - f);
      for (int s = 1; s <= ps_max; ++s) {
        const long long wg = (s + f + nw - 1) / nw;
        const long long rounds = (items * wg + resident - 1) / resident;
        const long long cost = rounds * (std::max<long long>(4LL * ((max_pages + s - 1) / s), f16) + 4);
        if (best < 0 || cost < best || (cost == best && s > ps)) {  // ties: more splits
          best = cost;
          ps = s;
          n16 = f;
        }
      }
    }
    // The fp16 pieces spread over the page splits, last split first.  The plan sees only the
    // capacity (max_pages); measured side by side at 64 pages with capacity 65 (call us, pieces
    // spread against an fp16 split of their own): Qwen3-8B B = 32 54.4 against 57.8, Llama-3.1-8B
    // B = 110 166.2 against 183.1, Qwen3-32B B = 32 (256 pages) 207.9 against 217.4; at 63 pages
    // with capacity 64 Qwen3-8B takes 55.9 against 54.4 and B = 1 at 32K 19.0 against 17.8 (the
    // cost model keeps the fp16 split there).  The larger slices must still fit a workgroup; the
    // resident workgroups are counted with them.
    if ((nw == 1 && items >= 128) || (nw > 1 && nw * fold_wave <= device_lds_per_block())) {
      const long long resident_f =
          (long long)dispatch(c, BlocksPerCu{nw * fold_wave, 64 * nw}) * device_cus();
      for (int s = 1; s <= std::min(max_pages, kMergeSplits * nw); ++s) {
        const long long wg = (s + nw - 1) / nw;
        const long long rounds = (items * wg + resident_f - 1) / resident_f;
        long long wave = 0;
        for (int w = 0; w < s; ++w) {
          const int pgs = (max_pages - 1 - w) / s + 1;  // w < s <= max_pages
          const int i = s - 1 - w;
          const int pcs = i < pieces ? (pieces - 1 - i) / s + 1 : 0;
          wave = std::max<long long>(wave, 4LL * pgs + kPieceCost * pcs);
        }
        const long long cost = rounds * (wave + 4);
        if (cost < best) {
          best = cost;
          ps = s;
          n16 = 0;
          fold = pieces;
        }
      }
    }
  }
  p.page_splits = ps;
  p.n16 = n16;
  p.fold16 = fold;
  p.pages_per_split = ps > 0 ? (max_pages + ps - 1) / ps : 0;
  p.splits = (ps + n16 + nw - 1) / nw;
  if (fold) {
    p.lds_wave = fold_wave;
    p.lds_bytes = (size_t)nw * p.lds_wave;
  }
  const size_t per = (size_t)items * p.splits * ng;
  const size_t o_bytes = (per * c.d * sizeof(float) + 255) & ~(size_t)255;
  p.ws_bytes = o_bytes + ((per * 2 * sizeof(float) + 255) & ~(size_t)255);
  return p;
}

struct Launch {
  const DecodePlan& p;
  int B;
  const pnmix_cfg& c;
  const DecodeArgs& a;
  hipStream_t stream;
  template <int D, int NT, int KG, int KH, bool PG>
  hipError_t split_kernel() const {
    const hipError_t la = allow_lds<D, NT, KG, KH, PG>(p.lds_bytes);
    if (la != hipSuccess) return la;
    hipLaunchKernelGGL((decode_kernel<D, NT, KG, KH, PG>), dim3(p.splits, B * c.H_kv),
                       dim3(64 * p.nw), p.lds_bytes, stream, a);
    return hipGetLastError();
  }
  template <int D, int NT, int KG, int KH>
  hipError_t run() const {
    // pages through a block table, or contiguous per (sequence, KV head)
    return a.table ? split_kernel<D, NT, KG, KH, true>() : split_kernel<D, NT, KG, KH, false>();
  }
};

// Merge launch: one workgroup of 256 per (sequence, query head); loads per lane and round: the
// lane's split count rounded up to a power of two (<= 8).
template <int D>
static hipError_t launch_merge(const DecodeArgs& a, int B, hipStream_t stream) {
  const int per_lane = (a.splits + (256 / (D / 4)) - 1) / (256 / (D / 4));
  const dim3 grid(B * a.H_q), block(256);
  if (per_lane <= 1)
    hipLaunchKernelGGL((decode_merge_kernel<D, 1>), grid, block, 0, stream, a);
  else if (per_lane <= 2)
    hipLaunchKernelGGL((decode_merge_kernel<D, 2>), grid, block, 0, stream, a);
  else if (per_lane <= 4)
    hipLaunchKernelGGL((decode_merge_kernel<D, 4>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, kMergeChunk>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const pnmix_cfg& c, int B, int max_pages, const uint16_t* q,
                         const uint16_t* k_sink, const uint16_t* v_sink, const uint8_t* k_pages,
                         const uint8_t* v_pages, const uint16_t* k_res, const uint16_t* v_res,
                         const pnmix_seq_len* lens, const uint32_t* mask, float sm_scale,
                         float* out, void* ws, hipStream_t stream, const int32_t* block_table,
                         int64_t n_blocks, const uint16_t* k_new, const uint16_t* v_new,
                         pnmix_seq_len* lens_out) {
  const DecodePlan p = decode_plan(c, B, max_pages);
  const int ng = c.H_q / c.H_kv;
  const size_t per = (size_t)B * c.H_kv * p.splits * ng;
  DecodeArgs a;
  a.q = q;
  a.k_sink = k_sink;
  a.v_sink = v_sink;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.table = block_table;
  a.n_blocks = n_blocks;
  a.k_new = k_new;
  a.v_new = v_new;
  a.lens_out = lens_out;
  a.k_res = k_res;
  a.v_res = v_res;
  a.lens = lens;
  a.mask = mask;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       ((per * c.d * sizeof(float) + 255) & ~(size_t)255));
  a.out = out;
  a.qscale = sm_scale * kLog2e;
  a.H_q = c.H_q;
  a.H_kv = c.H_kv;
  a.n_g = ng;
  a.pairing = c.pairing;
  a.n_hi = c.n_hi_pairs;
  a.n_sal = 2 * c.n_hi_pairs;
  a.G = c.G;
  a.KG = c.N / c.G;
  a.g_V = c.g_V;
  a.NGV = c.d / c.g_V;
  a.N_s = c.N_s;
  a.b_H = c.b_H;
  a.b_L = c.b_L;
  a.b_V = c.b_V;
  a.max_pages = max_pages;
  a.words = (c.d / 2 + 31) / 32;
  a.kpb = (int64_t)pnmix_k_page_bytes(&c);
  a.vpb = (int64_t)pnmix_v_page_bytes(&c);
  a.splits = p.splits;
  a.page_splits = p.page_splits;
  a.n16 = p.n16;
  a.fold16 = p.fold16;
  a.nw = p.nw;
  a.lds_T = decode_fast_path(c) ? (int)lds_T_bytes(c) : 0;
  a.lds_wave = (int)p.lds_wave;
  const hipError_t e = decode_fast_path(c) ? dispatch(c, Launch{p, B, c, a, stream})
                                           : launch_generic_split(a, c.d, B, p.lds_bytes, stream);
  if (e != hipSuccess) return e;
  switch (c.d) {
    case 32: return launch_merge<32>(a, B, stream);
    case 64: return launch_merge<64>(a, B, stream);
    default: return launch_merge<128>(a, B, stream);
  }
}

}  // namespace pnmix
