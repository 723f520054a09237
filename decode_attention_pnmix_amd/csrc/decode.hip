// decode.hip -- split-K GQA decode attention straight over the PN-Mix packed cache (gfx950).
//
// PN-Mix paper (arXiv 2610.19605), sec. 2, Eq. 1: causal GQA softmax attention; the
// kernel-implementation appendix: each decode step visits the sink region, the quantized region
// and the residual region, and the dequantized cache is never written back -- each quantized
// group is unpacked and dequantized on chip and consumed at once.  TriAxialKV fact sheet:
// flash-decoding splits merged by online log-sum-exp.
//
// Work decomposition.  The cache of one (sequence, KV head) is a list of blocks: block 0 holds
// the fp16 sinks, blocks 1..n_pages the packed pages, the last block the fp16 residual rows.
// A workgroup takes one (sequence, KV head, split) and a contiguous run of blocks; all n_g
// query heads of the GQA group are served from the same load of each page, so every packed
// byte is read once per step.  Inside a block, 32-token sub-tiles are dequantized into LDS
// (k = S q + Z with the page's fp16 S, Z), logits and an online softmax per head are kept in
// fp32, and the partial (m, l, o) of the split goes to the workspace.  A second kernel merges
// the splits: m = max m_j, l = sum e^(m_j - m) l_j, o = sum e^(m_j - m) o_j / l.
#include "common.h"
#include "kernels.h"

namespace pnmix {

constexpr int kDecThreads = 256;
constexpr int kSub = 32;       // tokens per LDS sub-tile
constexpr int kMaxG = 16;      // max query heads per KV head
constexpr int kMaxDim = 128;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_sink;
  const uint16_t* v_sink;
  const uint8_t* k_pages;
  const uint8_t* v_pages;
  const uint16_t* k_res;
  const uint16_t* v_res;
  const pnmix_seq_len* lens;
  const uint32_t* mask;
  float* part_o;   // [B*H_kv][splits][n_g][d]
  float* part_ml;  // [B*H_kv][splits][n_g][2]
  float sm_scale;
  int H_q, H_kv, d, pairing, n_hi, G, g_V, N_s, max_pages, words;
  int64_t kpb, vpb;
  int splits, bps;
};

__global__ void __launch_bounds__(kDecThreads) decode_split_kernel(DecodeArgs a) {
  __shared__ float qs[kMaxG][kMaxDim];
  __shared__ float Kd[kSub][kMaxDim + 1];
  __shared__ float Vd[kSub][kMaxDim];
  __shared__ float pl[kMaxG][kSub];
  __shared__ float alpha_s[kMaxG];
  __shared__ int srank[kMaxDim];

  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / a.H_kv;
  const int h = bh % a.H_kv;
  const int ng = a.H_q / a.H_kv;
  const int d = a.d;
  const int tid = threadIdx.x;
  constexpr int N = 128;  // page and residual length

  pnmix_seq_len L = a.lens[b];
  const int sink_len = min(max(L.sink_len, 0), a.N_s);
  const int n_pages = min(max(L.n_pages, 0), a.max_pages);
  const int res_len = min(max(L.res_len, 0), N);
  const int nblk = n_pages + 2;
  const int blk0 = split * a.bps;
  const int blk1 = min(blk0 + a.bps, nblk);

  const uint32_t* mrow = a.mask + (int64_t)bh * a.words;
  for (int i = tid; i < ng * d; i += blockDim.x) {
    const int hh = i / d, c = i % d;
    qs[hh][c] = h2f(a.q[((int64_t)b * a.H_q + h * ng + hh) * d + c]);
  }
  for (int c = tid; c < d; c += blockDim.x) srank[c] = salient_rank(mrow, c, d, a.pairing, a.n_hi);

  // thread-owned output accumulators: (head, channel) pairs i = tid + k * blockDim.x
  constexpr int kAcc = kMaxG * kMaxDim / kDecThreads;
  float acc[kAcc];
#pragma unroll
  for (int k = 0; k < kAcc; ++k) acc[k] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;  // valid in threads tid < ng (one head each)
  __syncthreads();

  const int n_sal = 2 * a.n_hi;
  for (int blk = blk0; blk < blk1; ++blk) {
    int ntok;
    const uint8_t* kp = nullptr;
    const uint8_t* vp = nullptr;
    const uint16_t* ksrc = nullptr;
    const uint16_t* vsrc = nullptr;
    if (blk == 0) {
      ntok = sink_len;
      ksrc = a.k_sink + (int64_t)bh * a.N_s * d;
      vsrc = a.v_sink + (int64_t)bh * a.N_s * d;
    } else if (blk == nblk - 1) {
      ntok = res_len;
      ksrc = a.k_res + (int64_t)bh * N * d;
      vsrc = a.v_res + (int64_t)bh * N * d;
    } else {
      ntok = N;
      kp = a.k_pages + ((int64_t)bh * a.max_pages + (blk - 1)) * a.kpb;
      vp = a.v_pages + ((int64_t)bh * a.max_pages + (blk - 1)) * a.vpb;
    }
    for (int st = 0; st < ntok; st += kSub) {
      const int nt = min(kSub, ntok - st);
      // ---- dequantize the sub-tile into LDS
      for (int i = tid; i < nt * d; i += blockDim.x) {
        const int t = i / d, c = i % d;
        const int tt = st + t;
        float kv, vv;
        if (kp) {
          const uint8_t* lo = kp;
          const uint8_t* hi = kp + N * d / 8;
          const uint16_t* S = reinterpret_cast<const uint16_t*>(hi + N * n_sal / 4);
          const uint16_t* Z = S + (N / a.G) * d;
          uint32_t code = (lo[(tt >> 3) * d + c] >> (tt & 7)) & 1u;
          const int r = srank[c];
          if (r >= 0) code |= ((hi[(tt >> 2) * n_sal + r] >> (2 * (tt & 3))) & 3u) << 1;
          const int g = tt / a.G;
          kv = h2f(S[g * d + c]) * (float)code + h2f(Z[g * d + c]);
          const int ngv = d / a.g_V;
          const uint16_t* VS = reinterpret_cast<const uint16_t*>(vp + N * d / 4);
          const uint16_t* VZ = VS + N * ngv;
          const uint32_t vcode =
              (vp[((tt >> 4) * (d / 4) + (c >> 2)) * 16 + (tt & 15)] >> (2 * (c & 3))) & 3u;
          const int gv = c / a.g_V;
          vv = h2f(VS[tt * ngv + gv]) * (float)vcode + h2f(VZ[tt * ngv + gv]);
        } else {
          kv = h2f(ksrc[(int64_t)tt * d + c]);
          vv = h2f(vsrc[(int64_t)tt * d + c]);
        }
        Kd[t][c] = kv;
        Vd[t][c] = vv;
      }
      __syncthreads();
      // ---- logits
      for (int i = tid; i < ng * nt; i += blockDim.x) {
        const int hh = i / nt, t = i % nt;
        float s = 0.0f;
        for (int c = 0; c < d; ++c) s += qs[hh][c] * Kd[t][c];
        pl[hh][t] = s * a.sm_scale;
      }
      __syncthreads();
      // ---- online softmax, one thread per head
      if (tid < ng) {
        float mx = m_run;
        for (int t = 0; t < nt; ++t) mx = fmaxf(mx, pl[tid][t]);
        const float al = expf(m_run - mx);  // m_run = -inf on the first tile: al = 0
        float sum = 0.0f;
        for (int t = 0; t < nt; ++t) {
          const float p = expf(pl[tid][t] - mx);
          pl[tid][t] = p;
          sum += p;
        }
        l_run = l_run * al + sum;
        m_run = mx;
        alpha_s[tid] = al;
      }
      __syncthreads();
      // ---- o = o * alpha + P V
#pragma unroll
      for (int k = 0; k < kAcc; ++k) {
        const int i = tid + k * kDecThreads;
        if (i < ng * d) {
          const int hh = i / d, c = i % d;
          float s = acc[k] * alpha_s[hh];
          for (int t = 0; t < nt; ++t) s += pl[hh][t] * Vd[t][c];
          acc[k] = s;
        }
      }
      __syncthreads();
    }
  }
  // ---- partials of this split
  const int64_t pbase = ((int64_t)bh * a.splits + split) * ng;
#pragma unroll
  for (int k = 0; k < kAcc; ++k) {
    const int i = tid + k * kDecThreads;
    if (i < ng * d) a.part_o[pbase * d + i] = acc[k];
  }
  if (tid < ng) {
    a.part_ml[(pbase + tid) * 2 + 0] = m_run;
    a.part_ml[(pbase + tid) * 2 + 1] = l_run;
  }
}

__global__ void __launch_bounds__(128) decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           float* __restrict__ out, int H_q,
                                                           int H_kv, int d, int splits) {
  const int bhq = blockIdx.x;  // b * H_q + hq
  const int b = bhq / H_q;
  const int hq = bhq % H_q;
  const int ng = H_q / H_kv;
  const int h = hq / ng, hh = hq % ng;
  const int64_t bh = (int64_t)b * H_kv + h;
  float m = -INFINITY;
  for (int s = 0; s < splits; ++s) m = fmaxf(m, part_ml[((bh * splits + s) * ng + hh) * 2]);
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    float l = 0.0f, o = 0.0f;
    for (int s = 0; s < splits; ++s) {
      const int64_t p = (bh * splits + s) * ng + hh;
      const float ms = part_ml[p * 2];
      if (ms == -INFINITY) continue;  // empty split
      const float w = expf(ms - m);
      l += w * part_ml[p * 2 + 1];
      o += w * part_o[p * d + c];
    }
    out[(int64_t)bhq * d + c] = l > 0.0f ? o / l : 0.0f;
  }
}

DecodePlan decode_plan(const pnmix_cfg& c, int B, int max_pages) {
  DecodePlan p;
  const int nblk = max_pages + 2;
  const long long items = (long long)B * c.H_kv;
  // aim for >= 2048 workgroups (8 per CU) while keeping >= 4 blocks per split
  int splits = (int)((2048 + items - 1) / items);
  splits = max(1, min(splits, (nblk + 3) / 4));
  p.blocks_per_split = (nblk + splits - 1) / splits;
  p.splits = (nblk + p.blocks_per_split - 1) / p.blocks_per_split;
  const int ng = c.H_q / c.H_kv;
  const size_t per = (size_t)items * p.splits * ng;
  size_t o_bytes = (per * c.d * sizeof(float) + 255) & ~(size_t)255;
  p.ws_bytes = o_bytes + ((per * 2 * sizeof(float) + 255) & ~(size_t)255);
  return p;
}

hipError_t launch_decode(const pnmix_cfg& c, int B, int max_pages, const uint16_t* q,
                         const uint16_t* k_sink, const uint16_t* v_sink, const uint8_t* k_pages,
                         const uint8_t* v_pages, const uint16_t* k_res, const uint16_t* v_res,
                         const pnmix_seq_len* lens, const uint32_t* mask, float sm_scale,
                         float* out, void* ws, hipStream_t stream) {
  const DecodePlan p = decode_plan(c, B, max_pages);
  const int ng = c.H_q / c.H_kv;
  const size_t per = (size_t)B * c.H_kv * p.splits * ng;
  DecodeArgs a;
  a.q = q;
  a.k_sink = k_sink;
  a.v_sink = v_sink;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.k_res = k_res;
  a.v_res = v_res;
  a.lens = lens;
  a.mask = mask;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                       ((per * c.d * sizeof(float) + 255) & ~(size_t)255));
  a.sm_scale = sm_scale;
  a.H_q = c.H_q;
  a.H_kv = c.H_kv;
  a.d = c.d;
  a.pairing = c.pairing;
  a.n_hi = c.n_hi_pairs;
  a.G = c.G;
  a.g_V = c.g_V;
  a.N_s = c.N_s;
  a.max_pages = max_pages;
  a.words = (c.d / 2 + 31) / 32;
  a.kpb = (int64_t)pnmix_k_page_bytes(&c);
  a.vpb = (int64_t)pnmix_v_page_bytes(&c);
  a.splits = p.splits;
  a.bps = p.blocks_per_split;
  hipLaunchKernelGGL(decode_split_kernel, dim3(p.splits, B * c.H_kv), dim3(kDecThreads), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(B * c.H_q), dim3(128), 0, stream, a.part_o,
                     a.part_ml, out, c.H_q, c.H_kv, c.d, p.splits);
  return hipGetLastError();
}

}  // namespace pnmix
