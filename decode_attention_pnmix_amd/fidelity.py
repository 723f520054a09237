"""Fidelity of the PN-Mix key cache against the fp16 cache it replaces (an analysis tool).

The PN-Mix paper (arXiv 2610.19605) judges a key-cache quantizer by how far the attention it
feeds moves from attention over the unquantized cache, and motivates the fixed mask by the
salient RoPE pairs chosen at prefill staying salient during decoding.  This module measures both
on given inputs:
* attention KL: the divergence of the attention weights over the packed cache (keys as the
  library reconstructs them, `pnmix_dequant_k_pages`) from those over the fp16 cache, the
  reproduction notes' "Attention KL";
* decode output error: `pnmix_decode_attn` over the packed cache against softmax attention over
  the same fp16 keys and values in float32 (mean squared error, largest absolute error, relative
  L2 error, cosine similarity per query head), and the sink-key error (0: sinks stay fp16);
* saliency overlap: the Jaccard index, per (sequence, KV head), of the pair mask the prefill
  tokens select and the mask the same score (`pnmix_score_prefill`, Eq. 6) selects on a window of
  later tokens; and the paper's per-(t, s) decode-time overlap and Jaccard (Figure 4, Table 11):
  the prefill mask against the top pairs of every decoding-time query-key pair, by pair-norm
  product or by absolute pair dot product, over consecutive ranges of decoding steps;
* the online-reselection ablation: pages quantized with masks re-chosen from the statistics
  accumulated up to each page, against the fixed prefill mask, with the per-page index bytes
  that re-choosing costs.
With r = 0 every key channel is 1-bit and with r = 1 every channel is 3-bit (uniform per-channel
min-max quantization of the keys), so running the same inputs at r = 0, the configured r and
r = 1 places PN-Mix between the two uniform key caches.  The packed cache comes from the
library's kernels; the references, divergences and overlaps are plain torch arithmetic.

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


def attention_logits_packed(cache: PNMixLayerCache, q: torch.Tensor) -> torch.Tensor:
    """Logits q . k^ * sm_scale over every cached token (sinks, pages, residual) of the packed
    cache, the keys as the library reconstructs them (pnmix_dequant_k_pages: S code + Z with the
    stored fp16 S, Z; the fp16 sinks and residual rows as they are), float64
    [B][H_q][tokens].  All sequences of the cache hold the same lengths."""
    cfg = cache.cfg
    B, H_kv, d = cache.B, cfg.H_kv, cfg.d
    s, n_p, r = cache.sink_len, cache.n_pages, cache.res_len
    parts = [cache.k_sink[:, :, :s].double()]
    if n_p:
        pages = cache.k_pages[:, :n_p].reshape(B * n_p * H_kv, -1).contiguous()
        rows = cache.mask.unsqueeze(1).expand(B, n_p, H_kv, -1).reshape(B * n_p * H_kv, -1)
        kx = L.pnmix_dequant_k_pages(cfg, pages, rows.contiguous())  # [B n_p H][N][d]
        kx = kx.view(B, n_p, H_kv, cfg.N, d).permute(0, 2, 1, 3, 4).reshape(B, H_kv, n_p * cfg.N, d)
        parts.append(kx.double())
    parts.append(cache.k_res[:, :, :r].double())
    kall = torch.cat(parts, dim=2)  # [B][H_kv][T][d]
    return _logits(q, kall, cache.sm_scale)


def _logits(q: torch.Tensor, k: torch.Tensor, sm_scale: float) -> torch.Tensor:
    B, H_q, d = q.shape
    H_kv = k.shape[1]
    ng = H_q // H_kv
    qf = q.double().reshape(B, H_kv, ng, d)
    lg = torch.matmul(qf, k.double().transpose(2, 3).contiguous()) * sm_scale  # [B][H_kv][ng][T]
    return lg.reshape(B, H_q, -1)


def attention_kl(ref_logits: torch.Tensor, logits: torch.Tensor) -> torch.Tensor:
    """KL(softmax(ref) || softmax(logits)) along the last axis, float64: the attention-weight
    divergence the PN-Mix paper uses to judge a key quantizer (the reproduction notes report it
    as "Attention KL").  Returns one value per leading index."""
    lp = torch.log_softmax(ref_logits.double(), dim=-1)
    lq = torch.log_softmax(logits.double(), dim=-1)
    return (lp.exp() * (lp - lq)).sum(-1)


def _pair_view(x: torch.Tensor, pairing: int) -> torch.Tensor:
    """[..., d] -> [..., d/2, 2]: the two channels of every RoPE pair."""
    d = x.shape[-1]
    if pairing == L.PAIRS_ADJACENT:
        return x.reshape(*x.shape[:-1], d // 2, 2)
    return torch.stack([x[..., : d // 2], x[..., d // 2:]], dim=-1)


def _top_set(score: torch.Tensor, n_hi: int) -> torch.Tensor:
    """Boolean [..., n_pairs]: the n_hi pairs of largest score, ties to the lower pair index (the
    selection rule of the prefill mask)."""
    order = torch.sort(score, dim=-1, descending=True, stable=True).indices[..., :n_hi]
    top = torch.zeros_like(score, dtype=torch.bool)
    return top.scatter_(-1, order, True)


def mask_bits(mask: torch.Tensor, n_pairs: int) -> torch.Tensor:
    """[..., words] uint32 patterns (held as int32) -> boolean [..., n_pairs]."""
    bits = torch.arange(32, device=mask.device, dtype=torch.int64)
    b = ((mask.to(torch.int64).unsqueeze(-1) >> bits) & 1).bool()
    return b.reshape(*mask.shape[:-1], -1)[..., :n_pairs]


def decode_time_overlap(mask: torch.Tensor, q_dec: torch.Tensor, k_dec: torch.Tensor,
                        pairing: int, n_hi: int, score: str = "pair_norm", bins: int = 4,
                        chunk: int = 64) -> dict:
    """How well the prefill mask predicts the salient pairs of each decoding-time query-key pair.
    PN-Mix paper, the Jaccard analysis of Figure 4 and the stability study of Table 11: for each
    decoding step t and each key s generated during decoding with s <= t, the decode-time salient
    set is the top-n_hi RoPE pairs of that (t, s) by
      score = "pair_norm": ||q_i^t|| ||k_i^s||   or   "abs_dot": |<q_i^t, k_i^s>|
    per query head and the KV head it reads; it is compared with the prefill mask of that KV
    head by overlap |A & M| / n_hi and Jaccard |A & M| / |A | M|, averaged over every eligible
    (t, s), query head and sequence, overall and over `bins` consecutive ranges of decoding steps
    (with the spread max - min over the bins).
      mask [B][H_kv][words]; q_dec [B][H_q][T_dec][d]; k_dec [B][H_kv][T_dec][d] (row j of both is
      decoding step j).  float64 arithmetic."""
    B, H_q, Td, d = q_dec.shape
    H_kv = k_dec.shape[1]
    ng = H_q // H_kv
    npairs = d // 2
    M = mask_bits(mask, npairs)  # [B][H_kv][np]
    qp = _pair_view(q_dec.double(), pairing)  # [B][H_q][Td][np][2]
    kp = _pair_view(k_dec.double(), pairing)
    qn, kn = qp.norm(dim=-1), kp.norm(dim=-1)
    ov_sum = torch.zeros(Td, dtype=torch.float64, device=q_dec.device)
    jac_sum = torch.zeros_like(ov_sum)
    cnt = torch.zeros_like(ov_sum)
    for t0 in range(0, Td, chunk):
        t1 = min(Td, t0 + chunk)
        for h in range(H_kv):
            Mh = M[:, h].view(B, 1, 1, 1, npairs)
            if score == "pair_norm":
                sc = qn[:, h * ng:(h + 1) * ng, t0:t1, None, :] * kn[:, h, None, None, :t1, :]
            else:
                sc = (qp[:, h * ng:(h + 1) * ng, t0:t1, None] * kp[:, h, None, None, :t1]).sum(-1).abs()
            A = _top_set(sc, n_hi)  # [B][ng][t][s][np]
            inter = (A & Mh).sum(-1).double()
            union = (A | Mh).sum(-1).double()
            ov = inter / max(n_hi, 1)
            jac = torch.where(union > 0, inter / union.clamp_min(1), torch.ones_like(union))
            causal = (torch.arange(t0, t1, device=q_dec.device).view(-1, 1) >=
                      torch.arange(t1, device=q_dec.device).view(1, -1))  # s <= t
            w = causal.view(1, 1, t1 - t0, t1).double()
            ov_sum[t0:t1] += (ov * w).sum((0, 1, 3))
            jac_sum[t0:t1] += (jac * w).sum((0, 1, 3))
            cnt[t0:t1] += w.sum((0, 1, 3)) * B * ng
    edges = [round(i * Td / bins) for i in range(bins + 1)]
    ov_bins = [float(ov_sum[a:b].sum() / cnt[a:b].sum()) for a, b in zip(edges, edges[1:]) if b > a]
    jac_bins = [float(jac_sum[a:b].sum() / cnt[a:b].sum()) for a, b in zip(edges, edges[1:]) if b > a]
    return {"score": score, "pairs": int(cnt.sum()), "overlap": float(ov_sum.sum() / cnt.sum()),
            "jaccard": float(jac_sum.sum() / cnt.sum()), "overlap_bins": ov_bins,
            "jaccard_bins": jac_bins, "overlap_spread": max(ov_bins) - min(ov_bins)}


def packed_vs_fp16(cache: PNMixLayerCache, q: torch.Tensor, k: torch.Tensor,
                   v: torch.Tensor) -> dict:
    """Attention over the packed cache against the fp16 cache it replaces, for decode queries q
    [B][H_q][d] at the end of the context k, v [B][H_kv][T][d]: attention KL (weights), output
    errors of the library's decode kernel, and the largest sink-key error (the sinks stay fp16,
    so it is 0)."""
    ref_lg = _logits(q, k.double(), cache.sm_scale)
    lg = attention_logits_packed(cache, q)
    kl = attention_kl(ref_lg, lg)
    out = cache.attend(q)
    ref = reference_attention(q, k, v, cache.sm_scale)
    s = cache.sink_len
    sink_err = float((cache.k_sink[:, :, :s].double() - k[:, :, :s].double()).abs().max()) if s else 0.0
    res = {"attn_kl_mean": float(kl.mean()), "attn_kl_max": float(kl.max()),
           "max_sink_key_error": sink_err}
    res.update(output_errors(out, ref))
    return res


def reselection_ablation(cfg: L.pnmix_cfg, q_all: torch.Tensor, k: torch.Tensor, P: int) -> dict:
    """The online-reselection ablation (Korean summary page, "전제와 한계": re-choosing the salient
    pairs per group from statistics accumulated during decoding scored lower than the fixed
    prefill mask and needs a per-group index stored and loaded).  For a context of T tokens with
    queries q_all [B][H_q][T][d] and keys k [B][H_kv][T][d] (fp16) and a P-token prompt:
      fixed:       every page quantized with the mask the prompt selects (PN-Mix);
      reselected:  page p quantized with the mask Eq. 6 selects on all tokens up to the end of
                   page p (the statistics available when the residual buffer holding it fills),
                   stored with the page (d/2 bits of index per page and KV head).
    Both caches are compared with the fp16 keys by the attention KL of the last query.  The
    library's decode kernel reads one mask per (sequence, KV head), so the reselected cache is
    evaluated on its dequantized pages (pnmix_dequant_k_pages with per-page mask rows)."""
    B, H_q, T, d = q_all.shape
    H_kv = cfg.H_kv
    s = min(T, cfg.N_s)
    n_pages = (T - s) // cfg.N
    words = L.pnmix_mask_words(cfg)
    kpb = L.pnmix_k_page_bytes(cfg)
    dev = k.device
    _, m_fixed = L.pnmix_score_prefill(cfg, q_all[:, :, :P].contiguous(), k[:, :, :P].contiguous(),
                                       want_sigma=False)
    masks_res = torch.empty(n_pages, B, H_kv, words, dtype=torch.int32, device=dev)
    for p in range(n_pages):
        end = s + (p + 1) * cfg.N
        _, masks_res[p] = L.pnmix_score_prefill(cfg, q_all[:, :, :end].contiguous(),
                                                k[:, :, :end].contiguous(), want_sigma=False)
    # pages [n_pages][B][H_kv], both mask choices
    src = k[:, :, s:s + n_pages * cfg.N].reshape(B, H_kv, n_pages, cfg.N, d)
    src = src.permute(2, 0, 1, 3, 4).contiguous()  # [p][b][h][N][d]
    n = n_pages * B * H_kv
    ptrs = [src.data_ptr() + i * cfg.N * d * 2 for i in range(n)]
    out = {}
    q_last = q_all[:, :, T - 1].contiguous()
    ref_lg = _logits(q_last, k.double(), float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32)))
    for name, rows in (("fixed", m_fixed.unsqueeze(0).expand(n_pages, -1, -1, -1)),
                       ("reselected", masks_res)):
        rows = rows.reshape(n, words).contiguous()
        pages = torch.zeros(n, kpb, dtype=torch.uint8, device=dev)
        jobs = L.page_jobs(ptrs, d, [pages.data_ptr() + i * kpb for i in range(n)], range(n), dev)
        L.pnmix_quantize_k_page(cfg, jobs, rows)
        kx = L.pnmix_dequant_k_pages(cfg, pages, rows).view(n_pages, B, H_kv, cfg.N, d)
        kx = kx.permute(1, 2, 0, 3, 4).reshape(B, H_kv, n_pages * cfg.N, d)
        kall = torch.cat([k[:, :, :s].double(), kx.double(), k[:, :, s + n_pages * cfg.N:].double()], 2)
        lg = _logits(q_last, kall, float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32)))
        kl = attention_kl(ref_lg, lg)
        out[name] = {"attn_kl_mean": float(kl.mean()), "attn_kl_max": float(kl.max())}
    same = (masks_res == m_fixed.unsqueeze(0)).all(-1).double().mean()
    out["pages"] = n_pages
    out["reselected_masks_equal_to_prefill"] = float(same)
    out["index_bytes_per_page_and_kv_head"] = words * 4
    out["index_bits_per_key_element"] = words * 32 / (cfg.N * d)
    out["extra_score_passes"] = n_pages
    return out


def main() -> None:
    import synth  # seeded synthetic inputs (repository root)

    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="tiny")
    ap.add_argument("--T", type=int, default=0, help="cached tokens (default: the workload's)")
    ap.add_argument("--B", type=int, default=0, help="sequences (default: min(B, 4))")
    ap.add_argument("--window", type=int, default=256, help="later tokens for the overlap")
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--decode-pairs", type=int, default=256,
                    help="decoding steps whose (t, s) pairs enter the decode-time overlap")
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
    # decode-time queries of every position after the prompt (the same law as the prompt's)
    q_all = synth.rope_tokens(sq, B, pos, w.d, w.pairing, w.rope_base, dev, w.name, args.layer,
                              "qall")
    for r in sorted({0.0, w.r, 1.0}):
        n_hi = L.pnmix_hi_pairs(r, w.d)
        cfg = L.make_cfg(w.H_q, w.H_kv, w.d, w.pairing, n_hi, G=w.G, b_H=w.b_H, b_L=w.b_L,
                         b_V=w.b_V, g_V=w.g_V, N_s=w.N_s, N=w.N)
        line = {"workload": w.name, "B": B, "T": T, "P": w.P, "r": r, "n_hi_pairs": n_hi}
        n_pages = max((T - min(T, w.N_s)) // w.N, 1)
        cache = PNMixLayerCache(cfg, B, n_pages, device=dev)
        cache.load_context(qp, k, v)
        line.update(packed_vs_fp16(cache, qd, k, v))
        jac = saliency_overlap(cfg, qp, k[:, :, :w.P], qw, kw)
        line.update({"overlap_window": win, "jaccard_mean": float(jac.mean()),
                     "jaccard_min": float(jac.min())})
        if 0 < n_hi < w.d // 2:
            dec = min(args.decode_pairs, T - w.P)
            for sc in ("pair_norm", "abs_dot"):
                line["decode_time_" + sc] = decode_time_overlap(
                    cache.mask, q_all[:, :, w.P:w.P + dec], k[:, :, w.P:w.P + dec], w.pairing,
                    n_hi, score=sc)
            line["reselection"] = reselection_ablation(cfg, q_all, k, w.P)
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
