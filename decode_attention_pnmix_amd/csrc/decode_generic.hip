// decode_generic.hip -- decode attention over the packed cache for every supported bit width.
//
// PN-Mix paper (arXiv 2610.19605), sec. 2, Eq. 1: GQA softmax attention at the decode
// position; kernel-implementation appendix: each step visits the sink region, the quantized
// region and the residual region, and a packed page is unpacked on chip and consumed, never
// written back dequantized; bit-width appendix and Table 14: the sweep over b_H, b_L in
// {1, 2, 3, 4} with the value cache at b_V = 16.
//
// The matrix-core kernel of decode.hip serves (b_H, b_L, b_V) = (3, 1, 2) with value groups of
// at least 32 channels.  This kernel serves every other supported setting, on the vector ALU in
// fp32.  One workgroup of 256 threads takes one (sequence, KV head, split).  A sequence's tokens
// come in chunks of N = 128: chunk 0 is the sink rows, chunks 1..n_pages the packed pages, the
// last chunk the residual rows; split s walks chunks s, s + S, s + 2S, ...  Per chunk:
//   1. the packed page bytes are copied to LDS (fp16 rows, and b_V = 16 value pages, are read
//      where they are);
//   2. thread (token t, channel half) forms qt . k_t over its half of the channels for every
//      query head of the GQA group, with k = S code + Z dequantized in registers (one fma), and
//      the two halves meet in LDS;
//   3. the 16 threads of query head h take the chunk's largest logit, rescale the running (m, l)
//      of the online softmax (log2 units: qt = q * sm_scale * log2 e) and turn logits into p;
//   4. thread (channel c, set of heads) accumulates sum_t p_t v_t with v = S code + Z.
// Partials (m, l, o) go to the workspace in the layout of decode.hip's split kernel, and its
// merge kernel folds them (and, for a fused append, places the new rows).
#include "common.h"
#include "decode_args.h"
#include "kernels.h"

namespace pnmix {

constexpr int kGThreads = 256;
constexpr int kGMaxNg = 16;

// LDS of one workgroup: scaled queries [16][d] f32, logits / p [16][N] f32, softmax state
// (m, l, alpha) [3][16] f32, salient rank [d] i32, then the K page bytes and the V page bytes
// (each rounded up to 16 bytes).
__host__ __device__ constexpr size_t round16(size_t x) { return (x + 15) & ~(size_t)15; }
__host__ __device__ constexpr size_t gen_lds_fixed(int d) {
  return round16((size_t)kGMaxNg * d * 4 + (size_t)kGMaxNg * kN * 4 + 3 * kGMaxNg * 4 +
                 (size_t)d * 4);
}
size_t generic_lds_bytes(const pnmix_cfg& c) {
  const size_t kpb = pnmix_k_page_bytes(&c);
  const size_t vpb = c.b_V == 16 ? 0 : pnmix_v_page_bytes(&c);
  return gen_lds_fixed(c.d) + round16(kpb) + round16(vpb);
}

__device__ __forceinline__ float f16_at(const uint8_t* p) {
  return h2f(*reinterpret_cast<const uint16_t*>(p));
}

template <int D, int NG>
__global__ void __launch_bounds__(kGThreads) decode_generic_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  float* qs = reinterpret_cast<float*>(lds);  // [16][D]
  float* lg = qs + kGMaxNg * D;               // [16][N]
  float* m_run = lg + kGMaxNg * kN;           // [16]
  float* l_run = m_run + kGMaxNg;
  float* alph = l_run + kGMaxNg;
  int* rank = reinterpret_cast<int*>(alph + kGMaxNg);  // [D]
  uint8_t* kb = lds + gen_lds_fixed(D);
  uint8_t* vb = kb + round16((size_t)a.kpb);

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int b = (int)(bh / a.H_kv), h = (int)(bh % a.H_kv);
  const int ng = a.n_g;
  const int bL = a.b_L, wH = a.b_H - a.b_L, bV = a.b_V;

  pnmix_seq_len L = a.lens[b];
  int new_kind = 2, new_row = 0;  // the fused append's row (kind 0 sink, 1 residual, 2 none)
  if (a.k_new) {
    append_slot(L, a.N_s, new_kind, new_row);
    if (new_kind == 0) L.sink_len = new_row + 1;
    if (new_kind == 1) L.res_len = new_row + 1;
  }
  const int sink_len = min(max(L.sink_len, 0), a.N_s);
  const int n_pages = min(max(L.n_pages, 0), a.max_pages);
  const int res_len = min(max(L.res_len, 0), kN);
  const int n_chunks = n_pages + 2;

  for (int i = tid; i < ng * D; i += kGThreads)
    qs[i] = h2f(a.q[((int64_t)b * a.H_q + (int64_t)h * ng) * D + i]) * a.qscale;
  for (int c = tid; c < D; c += kGThreads)
    rank[c] = salient_rank(a.mask + bh * a.words, c, D, a.pairing, a.n_hi);
  if (tid < kGMaxNg) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.0f;
  }
  // p.V ownership: channel c, heads hb, hb + HS, ...
  constexpr int HS = kGThreads / D;
  constexpr int NO = (NG + HS - 1) / HS;
  const int c_pv = tid % D, hb = tid / D;
  float o[NO];
#pragma unroll
  for (int k = 0; k < NO; ++k) o[k] = 0.0f;
  const int kOffS = kN * D * bL / 8 + kN * a.n_sal * wH / 8;  // K page: S after the planes
  const int kOffZ = kOffS + 2 * a.KG * D;
  const int vOffS = kN * D * bV / 8;                          // V page: S after the codes
  const int vOffZ = vOffS + 2 * a.NGV * kN;
  __syncthreads();

  for (int ci = split; ci < n_chunks; ci += a.splits) {
    const bool is_page = ci >= 1 && ci <= n_pages;
    const int kind = ci == 0 ? 0 : (is_page ? 1 : 2);  // sinks, page, residual
    const int T = kind == 0 ? sink_len : (kind == 1 ? kN : res_len);
    if (T == 0) continue;  // uniform over the workgroup
    // fp16 rows of this chunk (sinks or residual), and the fused append's row among them
    const uint16_t* krows = kind == 0 ? a.k_sink + bh * a.N_s * D : a.k_res + bh * kN * D;
    const uint16_t* vrows = kind == 0 ? a.v_sink + bh * a.N_s * D : a.v_res + bh * kN * D;
    const int t_new = (kind == 0 && new_kind == 0) || (kind == 2 && new_kind == 1) ? new_row : -1;
    const uint8_t* vpage = nullptr;
    if (is_page) {
      const int pg = ci - 1;
      int64_t blk;
      if (a.table) {
        blk = a.table[(int64_t)b * a.max_pages + pg];
        blk = min(max(blk, (int64_t)0), a.n_blocks - 1);
      } else {
        blk = (int64_t)b * a.max_pages + pg;
      }
      const uint8_t* kpage = a.k_pages + (blk * a.H_kv + h) * a.kpb;
      vpage = a.v_pages + (blk * a.H_kv + h) * a.vpb;
      for (int i = tid; i < (int)(a.kpb / 16); i += kGThreads)
        reinterpret_cast<uint4*>(kb)[i] = reinterpret_cast<const uint4*>(kpage)[i];
      if (bV != 16)
        for (int i = tid; i < (int)(a.vpb / 16); i += kGThreads)
          reinterpret_cast<uint4*>(vb)[i] = reinterpret_cast<const uint4*>(vpage)[i];
      __syncthreads();
    }

    // ---- logits: thread (token t, channel half)
    {
      const int t = tid & (kN - 1), half = tid >> 7;
      float acc[NG];
#pragma unroll
      for (int hh = 0; hh < NG; ++hh) acc[hh] = 0.0f;
      if (t < T) {
        const uint16_t* krow = t == t_new ? a.k_new + bh * D : krows + (int64_t)t * D;
        const int g = t / a.G;
        for (int c = half * (D / 2); c < (half + 1) * (D / 2); ++c) {
          float kv;
          if (is_page) {
            uint32_t code = plane_field(kb, D, bL, c, t);
            const int r = rank[c];
            if (wH > 0 && r >= 0) code |= plane_field(kb + kN * D * bL / 8, a.n_sal, wH, r, t) << bL;
            kv = __builtin_fmaf(f16_at(kb + kOffS + 2 * (g * D + c)), (float)code,
                                f16_at(kb + kOffZ + 2 * (g * D + c)));
          } else {
            kv = h2f(krow[c]);
          }
#pragma unroll
          for (int hh = 0; hh < NG; ++hh) acc[hh] = __builtin_fmaf(qs[hh * D + c], kv, acc[hh]);
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
#pragma unroll
      for (int k = 0; k < NO; ++k) {
        const int hh = hb + k * HS;
        if (hh < ng) o[k] *= alph[hh];
      }
      const int g = c_pv / a.g_V;
      const int e = bV == 16 ? 1 : 8 / bV;
      const uint32_t lmask = bV == 16 ? 0u : (1u << bV) - 1u;
      for (int t = 0; t < T; ++t) {
        float vv;
        if (is_page) {
          if (bV == 16) {
            vv = h2f(reinterpret_cast<const uint16_t*>(vpage)[(int64_t)t * D + c_pv]);
          } else {
            const uint32_t code = (vb[(c_pv / e) * kN + t] >> (bV * (c_pv % e))) & lmask;
            vv = __builtin_fmaf(f16_at(vb + vOffS + 2 * (g * kN + t)), (float)code,
                                f16_at(vb + vOffZ + 2 * (g * kN + t)));
          }
        } else {
          vv = h2f(t == t_new ? a.v_new[bh * D + c_pv] : vrows[(int64_t)t * D + c_pv]);
        }
#pragma unroll
        for (int k = 0; k < NO; ++k) {
          const int hh = hb + k * HS;
          if (hh < ng) o[k] = __builtin_fmaf(lg[hh * kN + t], vv, o[k]);
        }
      }
    }
    __syncthreads();  // LDS pages, logits and state are rewritten by the next chunk
  }

  // ---- partial of this split
  const int64_t pbase = (bh * a.splits + split) * ng;
#pragma unroll
  for (int k = 0; k < NO; ++k) {
    const int hh = hb + k * HS;
    if (hh < ng) a.part_o[(pbase + hh) * D + c_pv] = o[k];
  }
  if (tid < ng) {
    a.part_ml[(pbase + tid) * 2] = m_run[tid];
    a.part_ml[(pbase + tid) * 2 + 1] = l_run[tid];
  }
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, int B, size_t lds, hipStream_t stream) {
  const dim3 grid(a.splits, B * a.H_kv), block(kGThreads);
  const int ng = a.n_g;
  auto go = [&](auto kern) -> hipError_t {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, block, lds, stream, a);
    return hipGetLastError();
  };
  if (ng <= 1) return go(decode_generic_kernel<D, 1>);
  if (ng <= 2) return go(decode_generic_kernel<D, 2>);
  if (ng <= 4) return go(decode_generic_kernel<D, 4>);
  if (ng <= 8) return go(decode_generic_kernel<D, 8>);
  return go(decode_generic_kernel<D, 16>);
}

hipError_t launch_generic_split(const DecodeArgs& a, int d, int B, size_t lds, hipStream_t stream) {
  switch (d) {
    case 32: return launch_d<32>(a, B, lds, stream);
    case 64: return launch_d<64>(a, B, lds, stream);
    default: return launch_d<128>(a, B, lds, stream);
  }
}

}  // namespace pnmix
