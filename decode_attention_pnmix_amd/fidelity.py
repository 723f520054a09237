"""Fidelity of the PN-Mix key cache against the fp16 cache it replaces (an analysis tool).

The PN-Mix paper (arXiv 2610.19605) judges a key-cache quantizer by how far the attention it
feeds moves from attention over the unquantized cache, and motivates the fixed mask by the
salient RoPE pairs chosen at prefill staying salient during decoding.  This module measures both
on given inputs:
* decode output error: `pnmix_decode_attn` over the packed cache against softmax attention over
  the same fp16 keys and values in float32 (mean squared error, largest absolute error, relative
  L2 error, cosine similarity per query head);
* saliency overlap: the Jaccard index, per (sequence, KV head), of the pair mask the prefill
  tokens select and the mask the same score (`pnmix_score_prefill`, Eq. 6) selects on a window of
  later tokens.
With r = 0 every key channel is 1-bit and with r = 1 every channel is 3-bit (uniform per-channel
min-max quantization of the keys), so running the same inputs at r = 0, the configured r and
r = 1 places PN-Mix between the two uniform key caches.  The packed-cache outputs come from the
library's kernels; the fp16 reference is plain torch arithmetic.  The library returns attention
outputs, not attention weights, so no divergence between weight distributions is reported.

Command line (synthetic inputs of a named workload):
    python -m decode_attention_pnmix_amd.fidelity --workload tiny
    python -m decode_attention_pnmix_amd.fidelity --workload qwen3-8b-1L-32k --T 4096 --B 2
One JSON line per r.
"""
from __future__ import annotations

import argparse
import json

import torch

from . import _lib as L
from .cache import PNMixLayerCache


def reference_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        sm_scale: float) -> torch.Tensor:
    """softmax(q k^T sm_scale) v over every cached token, float32: q [B][H_q][d], k and v
    [B][H_kv][T][d]; query head h reads KV head floor(h / n_g)."""
    B, H_q, d = q.shape
    H_kv = k.shape[1]
    ng = H_q // H_kv
    qf = q.float().reshape(B, H_kv, ng, d)
    kt = k.float().transpose(2, 3).contiguous()  # [B][H_kv][d][T]
    p = torch.softmax(torch.matmul(qf, kt) * sm_scale, dim=-1)
    return torch.matmul(p, v.float().contiguous()).reshape(B, H_q, d)


def output_errors(out: torch.Tensor, ref: torch.Tensor) -> dict:
    """Error of out against ref, both [B][H_q][d]: MSE, max |diff|, ||diff|| / ||ref||, and the
    mean and smallest cosine similarity over (sequence, query head)."""
    o, r = out.double(), ref.double()
    diff = o - r
    cos = (o * r).sum(-1) / (o.norm(dim=-1) * r.norm(dim=-1)).clamp_min(1e-300)
    return {"mse": float((diff * diff).mean()), "max_abs": float(diff.abs().max()),
            "rel_l2": float(diff.norm() / r.norm().clamp_min(1e-300)),
            "cos_mean": float(cos.mean()), "cos_min": float(cos.min())}


def mask_jaccard(mask_a: torch.Tensor, mask_b: torch.Tensor) -> torch.Tensor:
    """|a & b| / |a | b| per (sequence, KV head) of two pair masks [B][H_kv][words] (uint32 bit
    patterns held as int32); two empty masks count as identical (1)."""
    bits = torch.arange(32, device=mask_a.device, dtype=torch.int64)

    def unpack(m):
        return ((m.to(torch.int64).unsqueeze(-1) >> bits) & 1).bool()

    a, b = unpack(mask_a), unpack(mask_b)
    inter = (a & b).sum((-1, -2)).double()
    union = (a | b).sum((-1, -2)).double()
    return torch.where(union > 0, inter / union.clamp_min(1), torch.ones_like(union))


def decode_fidelity(cfg: L.pnmix_cfg, q_prompt: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    q_dec: torch.Tensor) -> dict:
    """Decode at the end of a T-token context (k, v [B][H_kv][T][d] fp16), mask scored on the
    prompt q_prompt [B][H_q][P][d] against k[:, :, :P]; q_dec [B][H_q][d] is the decode query.
    Returns the output errors of the packed cache against the fp16 cache."""
    B, _, T, _ = k.shape
    n_pages = max((T - min(T, cfg.N_s)) // cfg.N, 1)
    cache = PNMixLayerCache(cfg, B, n_pages, device=k.device)
    cache.load_context(q_prompt, k, v)
    out = cache.attend(q_dec)
    ref = reference_attention(q_dec, k, v, cache.sm_scale)
    torch.cuda.synchronize()
    return output_errors(out, ref)


def saliency_overlap(cfg: L.pnmix_cfg, q_prompt: torch.Tensor, k_prompt: torch.Tensor,
                     q_later: torch.Tensor, k_later: torch.Tensor) -> torch.Tensor:
    """Jaccard index per (sequence, KV head) of the masks the Eq. 6 score selects on the prompt
    tokens and on a window of later tokens (each [B][heads][tokens][d] fp16)."""
    _, m_pre = L.pnmix_score_prefill(cfg, q_prompt.contiguous(), k_prompt.contiguous(),
                                     want_sigma=False)
    _, m_dec = L.pnmix_score_prefill(cfg, q_later.contiguous(), k_later.contiguous(),
                                     want_sigma=False)
    return mask_jaccard(m_pre, m_dec)


def main() -> None:
    import synth  # seeded synthetic inputs (repository root)

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="tiny")
    ap.add_argument("--T", type=int, default=0, help="cached tokens (default: the workload's)")
    ap.add_argument("--B", type=int, default=0, help="sequences (default: min(B, 4))")
    ap.add_argument("--window", type=int, default=256, help="later tokens for the overlap")
    ap.add_argument("--layer", type=int, default=0)
    args = ap.parse_args()
    w = synth.WORKLOADS[args.workload]
    T = args.T or w.T
    B = args.B or min(w.B, 4)
    dev = "cuda"
    npairs = w.d // 2
    sq = synth.pair_scales(w.H_q, npairs, w.sigma_ln, dev, w.name, args.layer, "q")
    sk = synth.pair_scales(w.H_kv, npairs, w.sigma_ln, dev, w.name, args.layer, "k")
    pos = torch.arange(T, device=dev)
    k = synth.rope_tokens(sk, B, pos, w.d, w.pairing, w.rope_base, dev, w.name, args.layer, "k")
    v = synth.values(B, w.H_kv, T, w.d, dev, w.name, args.layer)
    qp = synth.rope_tokens(sq, B, pos[:w.P], w.d, w.pairing, w.rope_base, dev, w.name,
                           args.layer, "qpre")
    qd = synth.rope_tokens(sq, B, pos[T - 1:], w.d, w.pairing, w.rope_base, dev, w.name,
                           args.layer, "qdec")[:, :, 0].contiguous()
    win = min(args.window, T)
    qw = synth.rope_tokens(sq, B, pos[T - win:], w.d, w.pairing, w.rope_base, dev, w.name,
                           args.layer, "qwin")
    kw = k[:, :, T - win:].contiguous()
    for r in sorted({0.0, w.r, 1.0}):
        n_hi = L.pnmix_hi_pairs(r, w.d)
        cfg = L.make_cfg(w.H_q, w.H_kv, w.d, w.pairing, n_hi, G=w.G, b_H=w.b_H, b_L=w.b_L, b_V=w.b_V,
                         g_V=w.g_V,
                         N_s=w.N_s, N=w.N)
        line = {"workload": w.name, "B": B, "T": T, "P": w.P, "r": r, "n_hi_pairs": n_hi}
        line.update(decode_fidelity(cfg, qp, k, v, qd))
        jac = saliency_overlap(cfg, qp, k[:, :, :w.P], qw, kw)
        line.update({"overlap_window": win, "jaccard_mean": float(jac.mean()),
                     "jaccard_min": float(jac.min())})
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
