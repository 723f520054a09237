// decode_generic.hip -- decode attention over the packed cache for every supported bit width.
//
// PN-Mix paper (arXiv 2610.19605), sec. 2, Eq. 1: GQA softmax attention at the decode
// position; kernel-implementation appendix: each step visits the sink region, the quantized
// region and the residual region, and a packed page is unpacked on chip and consumed, never
// written back dequantized; bit-width appendix and Table 14: the sweep over b_H, b_L in
// {1, 2, 3, 4} with the value cache at b_V = 16.
//
// The matrix-core kernel of decode.hip serves (b_H, b_L, b_V) = (3, 1, 2) with value groups of
// at least 32 channels.  This file serves every other supported setting.  One workgroup of 256
// threads (four waves) takes one (sequence, KV head, split).  A sequence's tokens come in
// chunks of N = 128: chunk 0 is the sink rows, chunks 1..n_pages the packed pages, the last
// chunk the residual rows; split s takes chunks s, s + S, s + 2S, ...  Partials (m, l, o) go to
// the workspace in the layout of decode.hip's split kernel, whose merge kernel folds them.
//
// Pages (decode_generic_mma_kernel), with qt = q * sm_scale * log2(e), keys k = S_gc code + Z_gc
// per (token group g, channel c), values v = S_tg code + Z_tg per (token t, value group g):
//   logit(h, t) = sum_c (qt_hc S_gc) code_tc + sum_c qt_hc Z_gc
//   o(h, c)    += sum_t (p_ht S_tg) code_tc + sum_t p_ht Z_tg       (b_V in {1, 2, 4})
//   o(h, c)    += sum_t p_ht v_tc                                    (b_V = 16)
// * The page is staged in LDS (the next page's bytes are loaded into registers while the
//   current one is computed).
// * q.K runs on v_mfma_i32_16x16x64_i8.  The products qt_hc S_gc (an upper-bit column r carries
//   the salient channel of rank r and the factor 2^b_L), rounded to fp32 and then to integers
//   below 2^30 with one power-of-two scale per (page, token group) from max|qt| and the group's
//   largest S, split into four balanced base-256 digits that fill a table T whose rows are
//   (head, digit) and whose columns are the LSB-plane channels, then the upper-plane ranks.  The B operand is the
//   key code of 16 tokens, cut out of the packed planes in registers: a w-bit field of token
//   8j + k sits at bits w k .. w k + w - 1 of the w bytes of octet j (across two bytes when
//   w = 3).  Integer accumulation is exact; the digit sums are combined in fp32.
// * p.V runs on the int8 matrix cores for b_V in {1, 2, 4}: x = p S_tg 2^sh below 2^22 (one
//   power-of-two scale per head and page, from the head's largest p and the page's largest
//   value scale) as three base-256 digits in a table W with rows (head, digit) per value group;
//   the B operand is the value code of one channel for 16 tokens.  For b_V = 16 it runs on
//   v_mfma_f32_16x16x32_f16 with p split into fp16 high and low parts (rows (head, part)) and
//   the fp16 value rows as stored.
// * The Z terms, the softmax and the state updates run on the vector ALU in fp32.
// Sink and residual rows (fp16) take the vector-ALU chunk code below, which is also the whole of
// decode_generic_valu_kernel: the fallback for configurations whose tables do not fit in 64 KiB
// of LDS (many query heads per KV head with small token groups and fp16 values).
#include "common.h"
#include "decode_args.h"
#include "kernels.h"

namespace pnmix {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kGThreads = 256;
constexpr int kGMaxNg = 16;

__host__ __device__ constexpr size_t round16(size_t x) { return (x + 15) & ~(size_t)15; }

__device__ __forceinline__ float f16_at(const uint8_t* p) {
  return h2f(*reinterpret_cast<const uint16_t*>(p));
}

// ------------------------------------------------------------------ vector-ALU chunk code

// One chunk of up to N tokens on the vector ALU.  kind 0: sink rows, 1: a packed page staged in
// LDS (kb, vb; b_V = 16 value rows read in place from vpage), 2: residual rows.
//   1. thread (token t, channel half) forms qt . k_t over its half of the channels for every
//      query head of the GQA group (a packed key dequantized in registers, one fma), and the two
//      halves meet in LDS;
//   2. the 16 threads of query head h take the chunk's largest logit, rescale the running
//      (m, l) of the online softmax and turn logits into p;
//   3. thread (channel c, set of heads) accumulates sum_t p_t v_t into its registers o.
template <int D, int NG>
struct ValuChunk {
  static constexpr int HS = kGThreads / D;           // threads per channel in p.V
  static constexpr int NO = (NG + HS - 1) / HS;      // heads per thread in p.V
  const DecodeArgs& a;
  int64_t bh;
  const float* qs;   // [n_g][D] scaled queries
  float* lg;         // [n_g][N] logits, then p
  float* m_run;
  float* l_run;
  float* alph;

  __device__ __forceinline__ void run(int kind, int T, const uint16_t* krows, const uint16_t* vrows, int t_new,
                      const uint8_t* kb, const uint8_t* vb, const uint8_t* vpage, const int* rank,
                      float (&o)[NO]) const {
    const int tid = threadIdx.x;
    const int ng = a.n_g;
    const bool is_page = kind == 1;
    const int bL = a.b_L, wH = a.b_H - a.b_L, bV = a.b_V;
    const int kOffS = kN * D * bL / 8 + kN * a.n_sal * wH / 8;  // K page: S after the planes
    const int kOffZ = kOffS + 2 * a.KG * D;
    const int vOffS = kN * D * bV / 8;                          // V page: S after the codes
    const int vOffZ = vOffS + 2 * a.NGV * kN;
    // ---- logits: thread (token t, channel half)
    {
      const int t = tid & (kN - 1), half = tid >> 7;
      float acc[NG];
#pragma unroll
      for (int hh = 0; hh < NG; ++hh) acc[hh] = 0.0f;
      if (is_page) {
        if (t < T) {
          const int g = t / a.G;
          for (int c = half * (D / 2); c < (half + 1) * (D / 2); ++c) {
            uint32_t code = plane_field(kb, D, bL, c, t);
            const int r = rank[c];
            if (wH > 0 && r >= 0) code |= plane_field(kb + kN * D * bL / 8, a.n_sal, wH, r, t) << bL;
            const float kv = __builtin_fmaf(f16_at(kb + kOffS + 2 * (g * D + c)), (float)code,
                                            f16_at(kb + kOffZ + 2 * (g * D + c)));
#pragma unroll
            for (int hh = 0; hh < NG; ++hh) acc[hh] = __builtin_fmaf(qs[hh * D + c], kv, acc[hh]);
          }
        }
      } else {
        // the lane's half row in 16-byte loads, all issued before the first use (a token past
        // the chunk reads the last row; its logit is replaced by -inf below)
        const int tc = min(t, T - 1);
        const uint16_t* krow = tc == t_new ? a.k_new + bh * D : krows + (int64_t)tc * D;
        uint4 kr[D / 16];
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
          kr[i] = *reinterpret_cast<const uint4*>(krow + half * (D / 2) + 8 * i);
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          const uint32_t wk[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int c = half * (D / 2) + 8 * i + e;
            const float kv = h2f((uint16_t)(wk[e >> 1] >> (16 * (e & 1))));
#pragma unroll
            for (int hh = 0; hh < NG; ++hh) acc[hh] = __builtin_fmaf(qs[hh * D + c], kv, acc[hh]);
          }
        }
      }
      if (half == 1) {
#pragma unroll
        for (int hh = 0; hh < NG; ++hh)
          if (hh < ng) lg[hh * kN + t] = acc[hh];
      }
      __syncthreads();
      if (half == 0) {
#pragma unroll
        for (int hh = 0; hh < NG; ++hh)
          if (hh < ng) lg[hh * kN + t] = t < T ? acc[hh] + lg[hh * kN + t] : -INFINITY;
      }
      __syncthreads();
    }
    // ---- online softmax: the 16 threads of head hh
    {
      const int hh = tid >> 4, l16 = tid & 15;
      if (hh < ng) {
        float cm = -INFINITY;
        for (int t = l16; t < kN; t += 16) cm = fmaxf(cm, lg[hh * kN + t]);
#pragma unroll
        for (int s = 8; s >= 1; s >>= 1) cm = fmaxf(cm, __shfl_xor(cm, s, 16));
        const float mo = m_run[hh];
        const float mn = fmaxf(mo, cm);  // finite: the chunk holds T >= 1 tokens
        float ps = 0.0f;
        for (int t = l16; t < kN; t += 16) {
          const float x = lg[hh * kN + t];
          const float p = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - mn);
          lg[hh * kN + t] = p;
          ps += p;
        }
#pragma unroll
        for (int s = 8; s >= 1; s >>= 1) ps += __shfl_xor(ps, s, 16);
        const float al = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
        if (l16 == 0) {
          alph[hh] = al;
          m_run[hh] = mn;
          l_run[hh] = l_run[hh] * al + ps;
        }
      }
      __syncthreads();
    }
    // ---- p.V: thread (channel c_pv, heads hb + k HS)
    {
      const int c_pv = tid % D, hb = tid / D;
#pragma unroll
      for (int k = 0; k < NO; ++k) {
        const int hh = hb + k * HS;
        if (hh < ng) o[k] *= alph[hh];
      }
      const int g = c_pv / a.g_V;
      const int e = bV == 16 ? 1 : 8 / bV;
      const uint32_t lmask = bV == 16 ? 0u : (1u << bV) - 1u;
      if (is_page) {
        for (int t = 0; t < T; ++t) {
          float vv;
          if (bV == 16) {
            vv = h2f(reinterpret_cast<const uint16_t*>(vpage)[(int64_t)t * D + c_pv]);
          } else {
            const uint32_t code = (vb[(c_pv / e) * kN + t] >> (bV * (c_pv % e))) & lmask;
            vv = __builtin_fmaf(f16_at(vb + vOffS + 2 * (g * kN + t)), (float)code,
                                f16_at(vb + vOffZ + 2 * (g * kN + t)));
          }
#pragma unroll
          for (int k = 0; k < NO; ++k) {
            const int hh = hb + k * HS;
            if (hh < ng) o[k] = __builtin_fmaf(lg[hh * kN + t], vv, o[k]);
          }
        }
      } else {
        // sixteen rows' values loaded before their use; a token past the chunk reads the last
        // row and weighs p = 0 (its logit is -inf)
        for (int t0 = 0; t0 < T; t0 += 16) {
          float vv[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tc = min(t0 + i, T - 1);
            vv[i] = h2f(tc == t_new ? a.v_new[bh * D + c_pv] : vrows[(int64_t)tc * D + c_pv]);
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
#pragma unroll
            for (int k = 0; k < NO; ++k) {
              const int hh = hb + k * HS;
              if (hh < ng) o[k] = __builtin_fmaf(lg[hh * kN + t0 + i], vv[i], o[k]);
            }
          }
        }
      }
    }
    __syncthreads();  // LDS pages, logits and state are rewritten by the next chunk
  }
};

// Cache lengths of sequence b as the kernel sees them, with a fused append's row counted in
// (new_kind 0: sink row new_row, 1: residual row new_row, 2: no row).
struct SeqView {
  int sink_len, n_pages, res_len, new_kind, new_row;
};
__device__ __forceinline__ SeqView seq_view(const DecodeArgs& a, int b) {
  pnmix_seq_len L = a.lens[b];
  SeqView v;
  v.new_kind = 2;
  v.new_row = 0;
  if (a.k_new) {
    append_slot(L, a.N_s, v.new_kind, v.new_row);
    if (v.new_kind == 0) L.sink_len = v.new_row + 1;
    if (v.new_kind == 1) L.res_len = v.new_row + 1;
  }
  v.sink_len = min(max(L.sink_len, 0), a.N_s);
  v.n_pages = min(max(L.n_pages, 0), a.max_pages);
  v.res_len = min(max(L.res_len, 0), kN);
  return v;
}

// The pool block of page pg of sequence b (block table entries clamped to the pool).
__device__ __forceinline__ int64_t page_block(const DecodeArgs& a, int b, int pg) {
  if (a.table) {
    int64_t blk = a.table[(int64_t)b * a.max_pages + pg];
    return min(max(blk, (int64_t)0), a.n_blocks - 1);
  }
  return (int64_t)b * a.max_pages + pg;
}

// Partial of this split: o [n_g][d] and (m, l) [n_g][2].
template <int D, int NG>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, int64_t bh, int split,
                                              const float (&o)[ValuChunk<D, NG>::NO],
                                              const float* m_run, const float* l_run) {
  using VC = ValuChunk<D, NG>;
  const int tid = threadIdx.x, ng = a.n_g;
  const int c_pv = tid % D, hb = tid / D;
  const int64_t pbase = (bh * a.splits + split) * ng;
#pragma unroll
  for (int k = 0; k < VC::NO; ++k) {
    const int hh = hb + k * VC::HS;
    if (hh < ng) a.part_o[(pbase + hh) * D + c_pv] = o[k];
  }
  if (tid < ng) {
    a.part_ml[(pbase + tid) * 2] = m_run[tid];
    a.part_ml[(pbase + tid) * 2 + 1] = l_run[tid];
  }
}

// LDS of the vector-ALU kernel: scaled queries [16][d] f32, logits / p [16][N] f32, softmax
// state (m, l, alpha) [3][16] f32, salient rank [d] i32, then the K page bytes and the V page
// bytes (each rounded up to 16 bytes).
__host__ __device__ constexpr size_t valu_lds_fixed(int d) {
  return round16((size_t)kGMaxNg * d * 4 + (size_t)kGMaxNg * kN * 4 + 3 * kGMaxNg * 4 +
                 (size_t)d * 4);
}
static size_t valu_lds_bytes(const pnmix_cfg& c) {
  const size_t kpb = pnmix_k_page_bytes(&c);
  const size_t vpb = c.b_V == 16 ? 0 : pnmix_v_page_bytes(&c);
  return valu_lds_fixed(c.d) + round16(kpb) + round16(vpb);
}

template <int D, int NG>
__global__ void __launch_bounds__(kGThreads) decode_generic_valu_kernel(DecodeArgs a) {
  using VC = ValuChunk<D, NG>;
  extern __shared__ __align__(16) uint8_t lds[];
  float* qs = reinterpret_cast<float*>(lds);  // [16][D]
  float* lg = qs + kGMaxNg * D;               // [16][N]
  float* m_run = lg + kGMaxNg * kN;           // [16]
  float* l_run = m_run + kGMaxNg;
  float* alph = l_run + kGMaxNg;
  int* rank = reinterpret_cast<int*>(alph + kGMaxNg);  // [D]
  uint8_t* kb = lds + valu_lds_fixed(D);
  uint8_t* vb = kb + round16((size_t)a.kpb);

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
  const int ng = a.n_g;
  const SeqView sv = seq_view(a, b);
  const int n_chunks = sv.n_pages + 2;

  for (int i = tid; i < ng * D; i += kGThreads)
    qs[i] = h2f(a.q[((int64_t)b * a.H_q + (int64_t)h * ng) * D + i]) * a.qscale;
  for (int c = tid; c < D; c += kGThreads)
    rank[c] = salient_rank(a.mask + bh * a.words, c, D, a.pairing, a.n_hi);
  if (tid < kGMaxNg) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.0f;
  }
  float o[VC::NO];
#pragma unroll
  for (int k = 0; k < VC::NO; ++k) o[k] = 0.0f;
  __syncthreads();
  const VC vc{a, bh, qs, lg, m_run, l_run, alph};

  for (int ci = split; ci < n_chunks; ci += a.splits) {
    const bool is_page = ci >= 1 && ci <= sv.n_pages;
    const int kind = ci == 0 ? 0 : (is_page ? 1 : 2);  // sinks, page, residual
    const int T = kind == 0 ? sv.sink_len : (kind == 1 ? kN : sv.res_len);
    if (T == 0) continue;  // uniform over the workgroup
    const uint16_t* krows = kind == 0 ? a.k_sink + bh * a.N_s * D : a.k_res + bh * kN * D;
    const uint16_t* vrows = kind == 0 ? a.v_sink + bh * a.N_s * D : a.v_res + bh * kN * D;
    const int t_new = (kind == 0 && sv.new_kind == 0) || (kind == 2 && sv.new_kind == 1) ? sv.new_row : -1;
    const uint8_t* vpage = nullptr;
    if (is_page) {
      const int64_t blk = page_block(a, b, ci - 1);
      const uint8_t* kpage = a.k_pages + (blk * a.H_kv + h) * a.kpb;
      vpage = a.v_pages + (blk * a.H_kv + h) * a.vpb;
      for (int i = tid; i < (int)(a.kpb / 16); i += kGThreads)
        reinterpret_cast<uint4*>(kb)[i] = reinterpret_cast<const uint4*>(kpage)[i];
      if (a.b_V != 16)
        for (int i = tid; i < (int)(a.vpb / 16); i += kGThreads)
          reinterpret_cast<uint4*>(vb)[i] = reinterpret_cast<const uint4*>(vpage)[i];
      __syncthreads();
    }
    vc.run(kind, T, krows, vrows, t_new, kb, vb, vpage, rank, o);
  }
  write_partial<D, NG>(a, bh, split, o, m_run, l_run);
}

// --------------------------------------------------------------------- matrix-core kernel

constexpr int kTRowPad = 16;       // T row padding: 16 rows of an A-operand read on distinct banks
constexpr int kWRow = kN + 16;     // W row stride (bytes)
constexpr int kPRow = 2 * kN + 16; // P row stride (bytes)
constexpr int kStBytes = 2432;     // softmax state, per-wave partials, scales, salient channels
constexpr int kZeroBytes = 256;    // a zero A-operand row
// y + 2^23 + 0x8080 (0 <= y < 2^23 - 0x8080) rounds y to an integer and leaves y + 0x8080 in the
// low 23 bits: bytes 0 and 1 xor 0x80 are y's balanced base-256 digits, byte 2 the top digit
constexpr float kTwo23b = 8421504.0f;

// LDS offsets (bytes) and page offsets of the matrix-core kernel, on the host (plan) and the
// device (the same arithmetic).
struct GLayout {
  int KSL, KSH, KS, TLB;                      // K-steps of 64 columns: LSB plane, upper plane
  int kOffH, kOffS, kOffZ, vOffS, vOffZ, VRS;  // page offsets; LDS row stride of fp16 values
  int qs, st, zero, kb, vb, u, pv;           // LDS regions of a page
  int vr, p16, pv16;                          // LDS regions of an fp16 row chunk (over kb..)
  int total;
};
__host__ __device__ inline GLayout glayout(int D, int ng, int KG, int NGV, int n_sal, int bL,
                                           int wH, int bV, int64_t kpb, int64_t vpb) {
  GLayout L;
  L.KSL = (D + 63) / 64;
  L.KSH = (wH > 0 && n_sal > 0) ? (n_sal + 63) / 64 : 0;
  L.KS = L.KSL + L.KSH;
  L.TLB = 64 * L.KS + kTRowPad;
  L.kOffH = kN * D * bL / 8;
  L.kOffS = L.kOffH + kN * n_sal * wH / 8;
  L.kOffZ = L.kOffS + 2 * KG * D;
  L.vOffS = bV == 16 ? 0 : kN * D * bV / 8;
  L.vOffZ = L.vOffS + 2 * NGV * kN;
  L.VRS = 2 * D + 8;  // 8 bytes of padding: the 4 token octets of an operand read hit 4 banks
  L.qs = 0;
  L.st = (int)round16((size_t)ng * D * 4);
  L.zero = L.st + kStBytes;
  L.kb = L.zero + kZeroBytes;
  // 64 bytes past each page: operand reads that run past a plane stay inside the buffer
  L.vb = L.kb + (int)round16((size_t)kpb) + 64;
  const int vbytes = bV == 16 ? kN * L.VRS : (int)round16((size_t)vpb) + 64;
  L.u = L.vb + (int)round16((size_t)vbytes);
  // region u: T (until the logits are done), then W or P plus the page's p.V sums
  const int tb = KG * 4 * ng * L.TLB;
  const int wt = (int)round16(bV == 16 ? (size_t)2 * ng * kPRow : (size_t)NGV * 3 * ng * kWRow);
  const int pvb = ng * D * 4;
  L.pv = L.u + wt;
  const int ub = tb > wt + pvb ? tb : wt + pvb;
  const int tp = L.u + (int)round16((size_t)ub);
  // fp16 row chunks: the value rows (row stride VRS), p halves, p.V sums, over the page regions
  L.vr = L.kb;
  L.p16 = L.vr + (int)round16((size_t)kN * L.VRS);
  L.pv16 = L.p16 + (int)round16((size_t)2 * ng * kPRow);
  const int tr = L.pv16 + (int)round16((size_t)pvb);
  L.total = tp > tr ? tp : tr;
  return L;
}
static GLayout glayout_cfg(const pnmix_cfg& c) {
  return glayout(c.d, c.H_q / c.H_kv, c.N / c.G, c.d / c.g_V, 2 * c.n_hi_pairs, c.b_L,
                 c.b_H - c.b_L, c.b_V, (int64_t)pnmix_k_page_bytes(&c),
                 (int64_t)pnmix_v_page_bytes(&c));
}
static GLayout glayout_args(const DecodeArgs& a, int d) {
  return glayout(d, a.n_g, a.KG, a.NGV, a.n_sal, a.b_L, a.b_H - a.b_L, a.b_V, a.kpb, a.vpb);
}
// the matrix-core kernel where its LDS fits in 64 KiB, else the vector-ALU kernel
static bool generic_mma(const pnmix_cfg& c) { return glayout_cfg(c).total <= 65536; }

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float p2i(int e) {  // 2^e, e in [-126, 127]
  return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}
// Lane moves inside a 16-lane row (quad_perm [1,0,3,2], [2,3,0,1], row_ror 4, row_ror 8: every
// lane reads a valid lane)
template <int CTRL>
__device__ __forceinline__ float rdpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, true));
}
__device__ __forceinline__ float rsum16(float x) {
  x = x + rdpp<0xB1>(x);
  x = x + rdpp<0x4E>(x);
  x = x + rdpp<0x124>(x);
  return x + rdpp<0x128>(x);
}
__device__ __forceinline__ float rmax16(float x) {
  x = fmaxf(x, rdpp<0xB1>(x));
  x = fmaxf(x, rdpp<0x4E>(x));
  x = fmaxf(x, rdpp<0x124>(x));
  return fmaxf(x, rdpp<0x128>(x));
}
typedef __amdgpu_buffer_rsrc_t grsrc_t;
// Buffer resource of `bytes` bytes at base: reads past the end return zero.
__device__ __forceinline__ grsrc_t g_rsrc(const void* base, int64_t bytes) {
  const int nb = (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nb, 0x00020000);
}
__device__ __forceinline__ v4u g_load16(grsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// maximum over the wave (every lane active): within 16-lane rows by DPP, then across the rows
template <int CTRL>
__device__ __forceinline__ uint32_t udpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, udpp<0xB1>(x));
  x = max(x, udpp<0x4E>(x));
  x = max(x, udpp<0x124>(x));
  x = max(x, udpp<0x128>(x));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(r0, r1), max(r2, r3));
}
// largest |x| of eight fp16 as its bit pattern (magnitudes order like their bits)
__device__ __forceinline__ uint32_t hmax8(const v4u& w) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = max(m, max(w[e] & 0x7FFFu, (w[e] >> 16) & 0x7FFFu));
  return m;
}
// 16 bytes of LDS at a 2-byte-aligned offset: the five dwords that cover them and a byte shift
__device__ __forceinline__ v4u lds16_a2(const uint8_t* lds, int off) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(lds + (off & ~3));
  const uint32_t sh = (uint32_t)off & 3u;
  const uint32_t d0 = p[0], d1 = p[1], d2 = p[2], d3 = p[3], d4 = p[4];
  return v4u{__builtin_amdgcn_alignbyte(d1, d0, sh), __builtin_amdgcn_alignbyte(d2, d1, sh),
             __builtin_amdgcn_alignbyte(d3, d2, sh), __builtin_amdgcn_alignbyte(d4, d3, sh)};
}
// Codes of token 8 j + k for 16 consecutive columns of a w-bit plane ([N/8][w][stride] bytes),
// one byte each: the field at bits w k .. w k + w - 1 of the octet's w bytes, taken from byte
// row i0 = (w k) / 8 at shift s = (w k) % 8 and, where it crosses into row i0 + 1 (w = 3), the
// rest from there.  Column offset c0; `aligned`: the rows start on 16 bytes.
__device__ __forceinline__ v4u plane_codes(const uint8_t* lds, int plane, int stride, int w, int j,
                                           int k, int c0, bool aligned) {
  const int pos = w * k, i0 = pos >> 3, s = pos & 7;
  const int off = plane + (j * w + i0) * stride + c0;
  const int lo = min(w, 8 - s);
  const uint32_t m0 = ((1u << lo) - 1u) * 0x01010101u;
  const v4u w0 = aligned ? *reinterpret_cast<const v4u*>(lds + off) : lds16_a2(lds, off);
  v4u r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (w0[e] >> s) & m0;
  if (w == 3) {  // uniform: only 3-bit fields cross a byte
    const uint32_t m1 = (((1u << w) - 1u) ^ ((1u << lo) - 1u)) * 0x01010101u;
    const v4u w1 = aligned ? *reinterpret_cast<const v4u*>(lds + off + stride)
                           : lds16_a2(lds, off + stride);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] |= (w1[e] << lo) & m1;
  }
  return r;
}

// Three waves per SIMD where that fits without spills: fp16 values with one head block (its
// LDS allows three workgroups per CU at d = 128; the compiler would otherwise take 170
// registers and two)
template <int D, int NHB, bool BV16>
__global__ void __launch_bounds__(kGThreads)
    __attribute__((amdgpu_waves_per_eu(BV16 && NHB == 1 ? 3 : 2)))
    decode_generic_mma_kernel(DecodeArgs a) {
  constexpr int NG = 4 * NHB;  // heads of the instantiation (n_g <= NG)
  using VC = ValuChunk<D, NG>;
  extern __shared__ __align__(16) uint8_t lds[];
  const int ng = a.n_g;
  const int bL = a.b_L, wH = a.b_H - a.b_L, bV = a.b_V;
  const int n_sal = a.n_sal, KG = a.KG, NGV = a.NGV;
  const GLayout L = glayout(D, ng, KG, NGV, n_sal, bL, wH, bV, a.kpb, a.vpb);
  float* qs = reinterpret_cast<float*>(lds + L.qs);  // [n_g][D] qt
  float* st = reinterpret_cast<float*>(lds + L.st);
  float* m_run = st;         // [16] running maximum (log2 units)
  float* l_run = st + 16;    // [16] running sum
  float* alph = st + 32;     // [16] rescale factor of this chunk
  float* mnew = st + 48;     // [16] maximum after this page
  float* shf = st + 64;      // [16] 2^-sh of this page's p.V fixed point
  float* wmax = st + 80;     // [4 waves][16] page maximum per wave
  float* wl = st + 144;      // [4][16] sum of p 2^sh per wave
  float* wz = st + 208;      // [4][16][4] sum of p 2^sh Z per wave and value group
  float* zk = st + 464;      // [4 groups][16] sum_c qt Z
  uint32_t* smaxk = reinterpret_cast<uint32_t*>(st + 528);  // [2][4] largest key S per group
  uint32_t* smaxv = reinterpret_cast<uint32_t*>(st + 536);  // [2] largest value S
  uint32_t* qmaxp = reinterpret_cast<uint32_t*>(st + 538);  // max |qt|
  int16_t* crank = reinterpret_cast<int16_t*>(st + 540);    // [128] channel of salient rank r
  float* pvb = reinterpret_cast<float*>(lds + L.pv);         // [n_g][D] this page's p.V

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, n = lane & 15, kq = lane >> 4;
  const int split = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
  const SeqView sv = seq_view(a, b);

  for (int i = tid; i < ng * D; i += kGThreads)
    qs[i] = h2f(a.q[((int64_t)b * a.H_q + (int64_t)h * ng) * D + i]) * a.qscale;
  if (tid < 128) crank[tid] = -1;
  if (tid < kZeroBytes / 4) reinterpret_cast<uint32_t*>(lds + L.zero)[tid] = 0u;
  if (tid < 16) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.0f;
  }
  if (tid < 8) smaxk[tid] = 0u;
  if (tid < 2) smaxv[tid] = 0u;
  if (tid == 0) *qmaxp = 0u;
  float o[VC::NO];
#pragma unroll
  for (int k = 0; k < VC::NO; ++k) o[k] = 0.0f;
  __syncthreads();
  for (int c = tid; c < D; c += kGThreads) {
    const int r = salient_rank(a.mask + bh * a.words, c, D, a.pairing, a.n_hi);
    if (r >= 0) crank[r] = (int16_t)c;
  }
  {
    float qm = 0.0f;
    for (int i = tid; i < ng * D; i += kGThreads) qm = fmaxf(qm, fabsf(qs[i]));
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) qm = fmaxf(qm, __shfl_xor(qm, s));
    if (lane == 0) atomicMax(qmaxp, fbits(qm));
  }
  __syncthreads();
  const float qmax = __builtin_bit_cast(float, *qmaxp);
  constexpr int NCT = D / 16;  // p.V column tiles of 16 channels

  // p.V over 128 fp16 value rows (LDS, row stride VRS, from byte offset vbase) with p split
  // into fp16 halves (rows (head, part) of stride kPRow from pbase): job (column tile ct, block
  // of 8 heads hb8) on v_mfma_f32_16x16x32_f16, K = 32 tokens per step; sums to pvbase [n_g][D]
  auto pv_fp16 = [&](int vbase, int pbase, int pvbase) {
    constexpr int NH8 = (NG + 7) / 8;
    float* pvo = reinterpret_cast<float*>(lds + pvbase);
    for (int job = wv; job < NCT * NH8; job += 4) {
      const int ct = job % NCT, hb8 = job / NCT;
      const int c = 16 * ct + n;
      const int hh = 8 * hb8 + (n >> 1), part = n & 1;
      const int prow = hh < ng ? 2 * hh + part : -1;
      v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        v8h bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 32 * ks + 8 * kq + e;
          bv[e] = *reinterpret_cast<const _Float16*>(lds + vbase + t * L.VRS + 2 * c);
        }
        const int ao = (prow < 0 ? L.zero : pbase + prow * kPRow) + 2 * (32 * ks + 8 * kq);
        const v8h av = *reinterpret_cast<const v8h*>(lds + ao);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
      }
      // lane (channel c, rows 4 kq + i): head 8 hb8 + 2 kq + i / 2, part i % 2
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int ho = 8 * hb8 + 2 * kq + jj;
        if (ho < ng) pvo[ho * D + c] = acc[2 * jj] + acc[2 * jj + 1];
      }
    }
  };
  // accumulators: o = o alpha + this chunk's p.V sums (thread (channel, heads) layout)
  auto o_update = [&](int pvbase) {
    const float* pvo = reinterpret_cast<const float*>(lds + pvbase);
    const int c_pv = tid % D, hb = tid / D;
#pragma unroll
    for (int k = 0; k < VC::NO; ++k) {
      const int hh = hb + k * VC::HS;
      if (hh < ng) o[k] = __builtin_fmaf(o[k], alph[hh], pvo[hh * D + c_pv]);
    }
  };

  // fp16 rows (sinks or residual, T <= 128 of them; row t_new from k_new / v_new): wave wv takes
  // tokens 32 wv .. 32 wv + 31.  q.K on v_mfma_f32_16x16x32_f16 straight from the key rows (A:
  // 16 tokens x 32 channels a step) and the fp16 queries (B: head = column; products exact in
  // fp32), the value rows staged in LDS for pv_fp16.  Tokens past T read row T - 1 and weigh
  // p = 0.
  constexpr int KS16 = D / 32;
  auto rows_chunk = [&](int T, const uint16_t* krows, const uint16_t* vrows, int t_new) {
    v4u qb[KS16];
    {
      const uint16_t* qrow = a.q + ((int64_t)b * a.H_q + (int64_t)h * ng + (n < ng ? n : 0)) * D;
#pragma unroll
      for (int ks = 0; ks < KS16; ++ks)
        qb[ks] = n < ng ? *reinterpret_cast<const v4u*>(qrow + 32 * ks + 8 * kq) : v4u{0, 0, 0, 0};
    }
    const int t0 = 32 * wv;
    const uint16_t* knew = a.k_new + bh * D;
    const uint16_t* vnew = a.v_new + bh * D;
    v4u ka[2][KS16];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = min(t0 + 16 * tt + n, T - 1);
      const uint16_t* kr = t == t_new ? knew : krows + (int64_t)t * D;
#pragma unroll
      for (int ks = 0; ks < KS16; ++ks) ka[tt][ks] = *reinterpret_cast<const v4u*>(kr + 32 * ks + 8 * kq);
    }
    // value rows t0 .. t0 + 31: 16-byte piece u = lane + 64 j is row u / (D / 8), piece u % (D / 8)
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const int u = lane + 64 * j, r = u / (D / 8), qd = u % (D / 8);
      const int t = min(t0 + r, T - 1);
      const v4u x = *reinterpret_cast<const v4u*>((t == t_new ? vnew : vrows + (int64_t)t * D) + 8 * qd);
      uint2* dst = reinterpret_cast<uint2*>(lds + L.vr + (t0 + r) * L.VRS + 16 * qd);
      dst[0] = make_uint2(x[0], x[1]);
      dst[1] = make_uint2(x[2], x[3]);
    }
    // logits: lane (head n, tokens t0 + 16 tt + 4 kq + i)
    float lv[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      v4f st = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS16; ++ks)
        st = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, ka[tt][ks]),
                                                    __builtin_bit_cast(v8h, qb[ks]), st, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lv[tt][i] = t0 + 16 * tt + 4 * kq + i < T ? st[i] * a.qscale : -INFINITY;
        mx = fmaxf(mx, lv[tt][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool ok = n < ng;
    if (kq == 0 && ok) wmax[16 * wv + n] = mx;
    __syncthreads();
    {
      const float mp = fmaxf(fmaxf(wmax[n], wmax[16 + n]), fmaxf(wmax[32 + n], wmax[48 + n]));
      const float mo = m_run[n];
      // finite: token 0 of wave 0 is a row (T >= 1); waves past T hold -inf
      const float mn = fmaxf(mo, mp);
      const float al = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
      if (wv == 0 && kq == 0 && ok) {
        mnew[n] = mn;
        shf[n] = 1.0f;
        alph[n] = al;
      }
      float ls = 0.0f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t hi[2], lo[2];
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(lv[tt][i] - mn);
          const float p1 = __builtin_amdgcn_exp2f(lv[tt][i + 1] - mn);
          ls += p0 + p1;
          const uint16_t h0 = f2h(p0), h1 = f2h(p1);
          hi[i / 2] = (uint32_t)h0 | (uint32_t)h1 << 16;
          lo[i / 2] = (uint32_t)f2h(p0 - h2f(h0)) | (uint32_t)f2h(p1 - h2f(h1)) << 16;
        }
        if (ok) {
          const int t = t0 + 16 * tt + 4 * kq;
          *reinterpret_cast<uint2*>(lds + L.p16 + 2 * n * kPRow + 2 * t) = make_uint2(hi[0], hi[1]);
          *reinterpret_cast<uint2*>(lds + L.p16 + (2 * n + 1) * kPRow + 2 * t) = make_uint2(lo[0], lo[1]);
        }
      }
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      if (kq == 0 && ok) wl[16 * wv + n] = ls;
    }
    __syncthreads();
    if (tid < ng) {
      m_run[tid] = mnew[tid];
      const float ls = (wl[tid] + wl[16 + tid]) + (wl[32 + tid] + wl[48 + tid]);
      l_run[tid] = __builtin_fmaf(l_run[tid], alph[tid], ls);
    }
    pv_fp16(L.vr, L.p16, L.pv16);
    __syncthreads();
    o_update(L.pv16);
    __syncthreads();  // the chunk's LDS is reused by what follows
  };

  // ---- sink rows (chunk 0)
  if (split == 0 && sv.sink_len > 0)
    rows_chunk(sv.sink_len, a.k_sink + bh * a.N_s * D, a.v_sink + bh * a.N_s * D,
               sv.new_kind == 0 ? sv.new_row : -1);

  // ---- pages (chunks 1 .. n_pages)
  const int S = a.splits;
  int pg = (split == 0 ? S : split) - 1;
  if (pg < sv.n_pages) {
    constexpr int KC = (5 * D + 255) / 256;  // 16-byte pieces per thread: K page <= 80 d bytes
    constexpr int VC16 = BV16 ? D / 16 : (64 * D + 2048 + 4095) / 4096;  // V page
    v4u rk[KC], rv[VC16];
    // The loads of a page go out unconditionally (through empty resources when there is no
    // page): a load under a branch would make the compiler wait for it where the paths meet.
    auto issue = [&](int p) {
      grsrc_t kr = g_rsrc(a.k_pages, 0), vr = g_rsrc(a.v_pages, 0);
      if (p >= 0) {
        const int64_t blk = page_block(a, b, p);
        kr = g_rsrc(a.k_pages + (blk * a.H_kv + h) * a.kpb, a.kpb);
        vr = g_rsrc(a.v_pages + (blk * a.H_kv + h) * a.vpb, a.vpb);
      }
#pragma unroll
      for (int j = 0; j < KC; ++j) rk[j] = g_load16(kr, 16u * (uint32_t)(tid + kGThreads * j));
#pragma unroll
      for (int j = 0; j < VC16; ++j) rv[j] = g_load16(vr, 16u * (uint32_t)(tid + kGThreads * j));
    };
    // Loaded page to LDS, with the largest key S per token group and the largest value S
    // (Largest scales: one LDS atomic per wave and group, from a wave reduction; atomics of many
    // lanes on one address serialise.)
    auto put = [&](int par) {
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const int off = 16 * (tid + kGThreads * j);
        if (off < a.kpb) *reinterpret_cast<v4u*>(lds + L.kb + off) = rk[j];
        const int w0 = 16 * (64 * wv + kGThreads * j);  // this wave's bytes [w0, w0 + 1024)
        if (w0 < L.kOffZ && w0 + 1024 > L.kOffS) {     // uniform
          for (int g = 0; g < KG; ++g) {
            const int g0 = L.kOffS + 2 * D * g;
            if (w0 < g0 + 2 * D && w0 + 1024 > g0) {
              const uint32_t m = wave_max_u32(off >= g0 && off < g0 + 2 * D ? hmax8(rk[j]) : 0u);
              if (lane == 0) atomicMax(&smaxk[4 * par + g], m);
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < VC16; ++j) {
        const int i = tid + kGThreads * j, off = 16 * i;
        if (off < a.vpb) {
          if constexpr (BV16) {
            const int t = i / (D / 8), qd = i % (D / 8);
            uint2* dst = reinterpret_cast<uint2*>(lds + L.vb + t * L.VRS + 16 * qd);
            dst[0] = make_uint2(rv[j][0], rv[j][1]);
            dst[1] = make_uint2(rv[j][2], rv[j][3]);
          } else {
            *reinterpret_cast<v4u*>(lds + L.vb + off) = rv[j];
          }
        }
        if constexpr (!BV16) {
          const int w0 = 16 * (64 * wv + kGThreads * j);
          if (w0 < L.vOffZ && w0 + 1024 > L.vOffS) {  // uniform
            const uint32_t m = wave_max_u32(off >= L.vOffS && off < L.vOffZ ? hmax8(rv[j]) : 0u);
            if (lane == 0) atomicMax(&smaxv[par], m);
          }
        }
      }
    };
    // 2^sigma of token group g: |qt S 2^sigma| (times 2^b_L on the upper plane) below 2^30
    const float hiw = L.KSH > 0 ? (float)(1 << bL) : 1.0f;
    auto sigma = [&](int par, int g) -> int {
      const float M = qmax * h2f((uint16_t)smaxk[4 * par + g]) * hiw;
      if (!(M > 0.0f) || !(M < INFINITY)) return 0;
      const int e = (int)((fbits(M) >> 23) & 0xFF) - 127;
      return min(max(29 - e, -126), 126);
    };

    issue(pg);
    put(0);
    // T columns of this thread (fixed for the call): the 4-column unit tc4 = tid % CW4 of the
    // rows of heads th0, th0 + ths, ... (ths = 256 / CW4 threads per unit; threads past ths * CW4
    // build none), in every token group; tchan = the unit's four channels (0xFF: none).
    const int CW4 = 16 * L.KS;  // 4-column units of a T row
    const int tc4 = tid % CW4, ths = kGThreads / CW4, th0 = tid / CW4;
    const bool thi = 4 * tc4 >= 64 * L.KSL;  // an upper-plane unit (factor 2^b_L)
    uint32_t tchan = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int col = 4 * tc4 + e, r = col - 64 * L.KSL;
      const int c = !thi ? (col < D ? col : -1) : (r < n_sal ? crank[r] : -1);
      tchan |= (uint32_t)(c < 0 ? 0xFF : c) << (8 * e);
    }
    __syncthreads();
    const int lgG = __builtin_ctz((uint32_t)a.G);
    const int lgE = BV16 ? 0 : 3 - __builtin_ctz((uint32_t)bV);  // log2 of codes per value byte
    const int lgGV = __builtin_ctz((uint32_t)a.g_V);
    const uint32_t vmask = BV16 ? 0u : ((1u << bV) - 1u) * 0x01010101u;
    for (int it = 0; pg < sv.n_pages; pg += S, ++it) {
      const int par = it & 1;
      const int nx = pg + S;
      issue(nx < sv.n_pages ? nx : -1);
      if (tid < 4) smaxk[4 * (par ^ 1) + tid] = 0u;
      if (tid == 4) smaxv[par ^ 1] = 0u;

      // ---- P1: digit table T [group][head, digit][column] and the key offsets' sums
      if (th0 < ths) {
        for (int g = 0; g < KG; ++g) {
          const float sc = p2i(sigma(par, g)) * (thi ? hiw : 1.0f);
          float svs[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = (tchan >> (8 * e)) & 0xFF;
            svs[e] = c != 0xFF ? f16_at(lds + L.kb + L.kOffS + 2 * (g * D + c)) : 0.0f;
          }
          for (int hh = th0; hh < ng; hh += ths) {
            uint32_t wd[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int c = (tchan >> (8 * e)) & 0xFF;
              const float qv = c != 0xFF ? qs[hh * D + c] * sc : 0.0f;
              // balanced digits of x (|x| < 2^30): byte d, read as int8, is digit d
              const int x = (int)__builtin_rintf(qv * svs[e]);
              wd[e] = ((uint32_t)x + 0x80808080u) ^ 0x80808080u;
            }
            // digit d of the four columns -> one dword of row (head, d)
            const uint32_t t01 = __builtin_amdgcn_perm(wd[1], wd[0], 0x05010400u);
            const uint32_t t23 = __builtin_amdgcn_perm(wd[3], wd[2], 0x05010400u);
            const uint32_t u01 = __builtin_amdgcn_perm(wd[1], wd[0], 0x07030602u);
            const uint32_t u23 = __builtin_amdgcn_perm(wd[3], wd[2], 0x07030602u);
            uint8_t* tr = lds + L.u + (g * 4 * ng + 4 * hh) * L.TLB + 4 * tc4;
            *reinterpret_cast<uint32_t*>(tr) = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
            *reinterpret_cast<uint32_t*>(tr + L.TLB) = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
            *reinterpret_cast<uint32_t*>(tr + 2 * L.TLB) = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
            *reinterpret_cast<uint32_t*>(tr + 3 * L.TLB) = __builtin_amdgcn_perm(u23, u01, 0x07060302u);
          }
        }
      }
      {
        // sum_c qt Z of head 15 - tid / 16 (a 16-lane row; D / 16 channels a lane) and every
        // group: the last waves, which build the fewest T rows
        constexpr int SL = D / 16;
        const int hh = 15 - (tid >> 4);
        if (hh < ng) {  // uniform over the row
          for (int g = 0; g < KG; ++g) {
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < SL; ++e) {
              const int c = SL * n + e;
              acc = __builtin_fmaf(qs[hh * D + c], f16_at(lds + L.kb + L.kOffZ + 2 * (g * D + c)), acc);
            }
            acc = rsum16(acc);
            if (n == 0) zk[16 * g + hh] = acc;
          }
        }
      }
      __syncthreads();

      // ---- P2: logits of this wave's 32 tokens (one token group: 32 divides G)
      const int g2 = (32 * wv) >> lgG;
      const float inv2 = p2i(-sigma(par, g2));
      float lgv[2][NHB];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 32 * wv + 16 * tt + n, j8 = t >> 3, k8 = t & 7;
        v4i acc[NHB];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) acc[hb] = v4i{0, 0, 0, 0};
        for (int ks = 0; ks < L.KS; ++ks) {
          const v4u bw = ks < L.KSL
                             ? plane_codes(lds, L.kb, D, bL, j8, k8, 64 * ks + 16 * kq, true)
                             : plane_codes(lds, L.kb + L.kOffH, n_sal, wH, j8, k8,
                                           64 * (ks - L.KSL) + 16 * kq, false);
          const v4i bi = __builtin_bit_cast(v4i, bw);
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            const int hh = 4 * hb + (n >> 2);
            const int row = hh >= ng ? -1 : g2 * 4 * ng + 4 * hh + (n & 3);
            const int ao = (row < 0 ? L.zero : L.u + row * L.TLB) + 64 * ks + 16 * kq;
            const v4i ai = *reinterpret_cast<const v4i*>(lds + ao);
            acc[hb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, bi, acc[hb], 0, 0, 0);
          }
        }
        // lane (token t, rows 4 kq + i): digit i of head 4 hb + kq; c[0] + 256 c[1] and
        // c[2] + 256 c[3] are exact in int32 (|c[i]| < 2^19)
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const v4i& c = acc[hb];
          const float x = __builtin_fmaf((float)(c[2] + (c[3] << 8)), 65536.0f, (float)(c[0] + (c[1] << 8)));
          lgv[tt][hb] = __builtin_fmaf(x, inv2, zk[16 * g2 + 4 * hb + kq]);
        }
      }
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const float mx = rmax16(fmaxf(lgv[0][hb], lgv[1][hb]));
        if (n == 0 && 4 * hb + kq < ng) wmax[16 * wv + 4 * hb + kq] = mx;
      }
      __syncthreads();

      // ---- P3: softmax of the page; p.V tables (W digits or P halves) and this wave's sums
      // byte selectors of the quad transpose: [x.b0, y.b0, x.b2, y.b2] (even lanes) or
      // [y.b1, x.b1, y.b3, x.b3] (odd), y the neighbour's word; then the same over lane pairs
      const uint32_t qsel1 = (n & 1) ? 0x03070105u : 0x06020400u;
      const uint32_t qsel2 = (n & 2) ? 0x03020706u : 0x05040100u;
      const float smv = BV16 ? 0.0f : h2f((uint16_t)smaxv[par]);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const int hh = 4 * hb + kq;
        const bool ok = hh < ng;  // uniform over the lane's 16-lane row
        const float mp = fmaxf(fmaxf(wmax[hh], wmax[16 + hh]), fmaxf(wmax[32 + hh], wmax[48 + hh]));
        const float mo = m_run[hh];
        const float mn = fmaxf(mo, mp);
        const float al = mo == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
        int sh = 0;
        if (!BV16) {
          const float top = __builtin_amdgcn_exp2f(mp - mn) * smv;
          if (top > 0.0f) sh = min(max(21 - ((int)((fbits(top) >> 23) & 0xFF) - 127), -126), 126);
        }
        const float msh = mn - (float)sh;
        if (wv == 0 && n == 0 && ok) {
          mnew[hh] = mn;
          shf[hh] = p2i(-sh);
          alph[hh] = al;
        }
        float ls = 0.0f, zs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 32 * wv + 16 * tt + n;
          const float pw = __builtin_amdgcn_exp2f(lgv[tt][hb] - msh);
          ls += pw;
          if constexpr (BV16) {
            if (ok) {
              const uint16_t hi = f2h(pw);
              const uint16_t lo = f2h(pw - h2f(hi));
              uint16_t* pr = reinterpret_cast<uint16_t*>(lds + L.u + 2 * hh * kPRow) + t;
              pr[0] = hi;
              pr[kPRow / 2] = lo;
            }
          } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              if (g >= NGV) break;
              const float sg = f16_at(lds + L.vb + L.vOffS + 2 * (g * kN + t));
              const float zg = f16_at(lds + L.vb + L.vOffZ + 2 * (g * kN + t));
              const uint32_t xb = fbits(__builtin_fmaf(pw, sg, kTwo23b)) ^ 0x8080u;
              // 4 x 4 byte transpose in the lane quad (tokens 4q .. 4q + 3): lane i gets digit i
              // of the four tokens, one dword of row (head, digit i)
              const uint32_t s1 = __builtin_amdgcn_perm(udpp<0xB1>(xb), xb, qsel1);
              const uint32_t dw = __builtin_amdgcn_perm(udpp<0x4E>(s1), s1, qsel2);
              if (ok && (n & 3) < 3)
                *reinterpret_cast<uint32_t*>(lds + L.u + (g * 3 * ng + 3 * hh + (n & 3)) * kWRow +
                                             (t & ~3)) = dw;
              zs[g] = __builtin_fmaf(pw, zg, zs[g]);
            }
          }
        }
        ls = rsum16(ls);
        if (n == 0 && ok) wl[16 * wv + hh] = ls;
        if constexpr (!BV16) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            if (g >= NGV) break;
            const float z = rsum16(zs[g]);
            if (n == 0 && ok) wz[4 * (16 * wv + hh) + g] = z;
          }
        }
      }
      __syncthreads();

      // ---- P4: state of the page's heads; p.V of the page into pvb
      if (tid < ng) {
        m_run[tid] = mnew[tid];
        const float ls = (wl[tid] + wl[16 + tid]) + (wl[32 + tid] + wl[48 + tid]);
        l_run[tid] = __builtin_fmaf(l_run[tid], alph[tid], ls * shf[tid]);
      }
      if constexpr (!BV16) {
        for (int job = wv; job < NCT * NHB; job += 4) {
          const int ct = job % NCT, hb = job / NCT;
          const int c = 16 * ct + n, g = (16 * ct) >> lgGV;
          const int mcol = c >> lgE, fs = bV * (c & ((1 << lgE) - 1));
          const int hh = 4 * hb + (n >> 2), dg = n & 3;
          const int row = (dg == 3 || hh >= ng) ? -1 : g * 3 * ng + 3 * hh + dg;
          v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const v4u wv4 = *reinterpret_cast<const v4u*>(lds + L.vb + mcol * kN + 64 * ks + 16 * kq);
            v4i bi;
#pragma unroll
            for (int e = 0; e < 4; ++e) bi[e] = (int)((wv4[e] >> fs) & vmask);
            const int ao = (row < 0 ? L.zero : L.u + row * kWRow) + 64 * ks + 16 * kq;
            const v4i ai = *reinterpret_cast<const v4i*>(lds + ao);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, bi, acc, 0, 0, 0);
          }
          const int ho = 4 * hb + kq;  // lane (channel c, rows 4 kq + i): digit i of head ho
          if (ho < ng) {
            const float x = __builtin_fmaf((float)acc[2], 65536.0f, (float)(acc[0] + (acc[1] << 8)));
            const float zb = (wz[4 * ho + g] + wz[4 * (16 + ho) + g]) +
                             (wz[4 * (32 + ho) + g] + wz[4 * (48 + ho) + g]);
            pvb[ho * D + c] = (x + zb) * shf[ho];
          }
        }
      } else {
        pv_fp16(L.vb, L.u, L.pv);
      }
      __syncthreads();

      // ---- P5: accumulators; the next page into LDS
      o_update(L.pv);
      if (nx < sv.n_pages) put(par ^ 1);
      __syncthreads();
    }
  }

  // ---- residual rows (chunk n_pages + 1)
  if ((sv.n_pages + 1) % S == split && sv.res_len > 0)
    rows_chunk(sv.res_len, a.k_res + bh * kN * D, a.v_res + bh * kN * D,
               sv.new_kind == 1 ? sv.new_row : -1);

  write_partial<D, NG>(a, bh, split, o, m_run, l_run);
}

size_t generic_lds_bytes(const pnmix_cfg& c) {
  return generic_mma(c) ? (size_t)glayout_cfg(c).total : valu_lds_bytes(c);
}

// The kernel instantiation for head dim D, n_g query heads per KV head, value width b_V and
// whether the matrix-core kernel's LDS fits (else the vector-ALU kernel), passed to f.
template <int D, class F>
static auto with_generic_kernel(int ng, int bV, bool mma, F&& f) {
  if (mma) {
    if (bV == 16) {
      if (ng <= 4) return f(decode_generic_mma_kernel<D, 1, true>);
      if (ng <= 8) return f(decode_generic_mma_kernel<D, 2, true>);
      return f(decode_generic_mma_kernel<D, 4, true>);
    }
    if (ng <= 4) return f(decode_generic_mma_kernel<D, 1, false>);
    if (ng <= 8) return f(decode_generic_mma_kernel<D, 2, false>);
    return f(decode_generic_mma_kernel<D, 4, false>);
  }
  if (ng <= 1) return f(decode_generic_valu_kernel<D, 1>);
  if (ng <= 2) return f(decode_generic_valu_kernel<D, 2>);
  if (ng <= 4) return f(decode_generic_valu_kernel<D, 4>);
  if (ng <= 8) return f(decode_generic_valu_kernel<D, 8>);
  return f(decode_generic_valu_kernel<D, 16>);
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, int B, size_t lds, hipStream_t stream) {
  const dim3 grid(a.splits, B * a.H_kv), block(kGThreads);
  return with_generic_kernel<D>(a.n_g, a.b_V, glayout_args(a, D).total <= 65536,
                                [&](auto kern) -> hipError_t {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, block, lds, stream, a);
    return hipGetLastError();
  });
}

hipError_t launch_generic_split(const DecodeArgs& a, int d, int B, size_t lds, hipStream_t stream) {
  switch (d) {
    case 32: return launch_d<32>(a, B, lds, stream);
    case 64: return launch_d<64>(a, B, lds, stream);
    default: return launch_d<128>(a, B, lds, stream);
  }
}

template <int D>
static int blocks_d(const pnmix_cfg& c, size_t lds) {
  return with_generic_kernel<D>(c.H_q / c.H_kv, c.b_V, generic_mma(c), [&](auto kern) -> int {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kGThreads, lds) != hipSuccess ||
        n <= 0) {
      (void)hipGetLastError();
      return 1;
    }
    return n;
  });
}

int generic_blocks_per_cu(const pnmix_cfg& c, size_t lds) {
  switch (c.d) {
    case 32: return blocks_d<32>(c, lds);
    case 64: return blocks_d<64>(c, lds);
    default: return blocks_d<128>(c, lds);
  }
}

}  // namespace pnmix
