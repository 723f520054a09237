"""Shared builders for the GPU parity tests: seeded inputs of one workload layer on the GPU,
the library's cache filled from them, and the oracle's own cache built from the same fp16 bits
(never from the library's output)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import decode_attention_pnmix_amd as P
import oracle
import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cfgs(w: synth.Workload):
    lc = P.make_cfg(w.H_q, w.H_kv, w.d, w.pairing, w.n_hi_pairs, G=w.G, b_H=w.b_H, b_L=w.b_L,
                    b_V=w.b_V, g_V=w.g_V, N_s=w.N_s, N=w.N)
    oc = oracle.Cfg(w.H_q, w.H_kv, w.d, w.pairing, w.n_hi_pairs, G=w.G, b_H=w.b_H, b_L=w.b_L,
                    b_V=w.b_V, g_V=w.g_V, N_s=w.N_s, N=w.N)
    return lc, oc


def layer_inputs(w: synth.Workload, layer: int, B: int, T: int, P_: int | None = None,
                 device="cuda"):
    """Post-RoPE prefill queries (P tokens), keys and values of positions [0, T), and the decode
    query at position T-1, all fp16 on `device`."""
    P_ = w.P if P_ is None else P_
    npairs = w.d // 2
    sq = synth.pair_scales(w.H_q, npairs, w.sigma_ln, device, w.name, layer, "q")
    sk = synth.pair_scales(w.H_kv, npairs, w.sigma_ln, device, w.name, layer, "k")
    k = synth.rope_tokens(sk, B, torch.arange(T, device=device), w.d, w.pairing, w.rope_base,
                          device, w.name, layer, "k")
    v = synth.values(B, w.H_kv, T, w.d, device, w.name, layer)
    qp = synth.rope_tokens(sq, B, torch.arange(P_, device=device), w.d, w.pairing, w.rope_base,
                           device, w.name, layer, "qpre")
    qd = synth.rope_tokens(sq, B, torch.tensor([T - 1], device=device), w.d, w.pairing,
                           w.rope_base, device, w.name, layer, "qdec")[:, :, 0].contiguous()
    return qp, k, v, qd


def fill_cache_bulk(w, lc, qp, k, v, T, max_pages=None):
    """Library cache holding tokens [0, T): prefill score on the first P tokens, sinks, bulk page
    quantization of every full page, fp16 residual."""
    B = k.shape[0]
    n_pages = (T - w.N_s) // w.N if T >= w.N_s else 0
    max_pages = max(n_pages, 1) if max_pages is None else max_pages
    c = P.PNMixLayerCache(lc, B, max_pages)
    c.prefill(qp, k[:, :, :qp.shape[2]].contiguous(), v[:, :, :qp.shape[2]].contiguous())
    # bulk: re-place everything from the full token range with the prefill mask
    s = min(T, w.N_s)
    c.k_sink.zero_()
    c.v_sink.zero_()
    c.k_sink[:, :, :s] = k[:, :, :s]
    c.v_sink[:, :, :s] = v[:, :, :s]
    if n_pages:
        kj, _ = c.page_jobs(k, s, 0, n_pages)
        _, vj = c.page_jobs(v, s, 0, n_pages)
        P.pnmix_quantize_k_page(lc, kj, c.mask)
        P.pnmix_quantize_v_page(lc, vj)
    a = s + n_pages * w.N
    rest = T - a
    c.k_res.zero_()
    c.v_res.zero_()
    c.k_res[:, :, :rest] = k[:, :, a:T]
    c.v_res[:, :, :rest] = v[:, :, a:T]
    c.sink_len, c.n_pages, c.res_len = s, n_pages, rest
    c._sync_lens()
    torch.cuda.synchronize()
    return c


def placement(w, T, online=False):
    """(sink_len, n_pages, res_len) of a cache holding T tokens.  Bulk placement packs every
    full page (residual 0..N-1 rows); the online policy attends before it quantizes, so in the
    step that fills the residual buffer attention sees N fp16 residual rows (1..N rows)."""
    s = min(T, w.N_s)
    if T <= w.N_s:
        return s, 0, 0
    n_pages = (T - s - 1) // w.N if online else (T - s) // w.N
    return s, n_pages, T - s - n_pages * w.N


def oracle_decode(w, oc, qp_b, k_b, v_b, qd_b, T, sm_scale, mask_b=None, threads=None,
                  online=False):
    """Oracle output [H_q][d] for one sequence from its fp16 inputs (host numpy uint16):
    its own score -> mask, its own page quantization, float64 attention."""
    if mask_b is None:
        _, _, _, mask_b = oracle.score_prefill(oc, qp_b, k_b[:, :qp_b.shape[1]])
    s, n_pages, _ = placement(w, T, online)
    mp = max(n_pages, 1)
    kp = np.zeros((w.H_kv, mp, oracle.k_page_bytes(oc)), np.uint8)
    vp = np.zeros((w.H_kv, mp, oracle.v_page_bytes(oc)), np.uint8)
    jobs = [(h, p) for h in range(w.H_kv) for p in range(n_pages)]

    def q1(job):
        h, p = job
        a = s + p * w.N
        kp[h, p] = oracle.quantize_k_page(oc, k_b[h, a:a + w.N], mask_b[h])
        vp[h, p] = oracle.quantize_v_page(oc, v_b[h, a:a + w.N])

    oracle.parallel_map(q1, jobs, threads)
    ks = np.zeros((w.H_kv, w.N_s, w.d), np.uint16)
    vs = np.zeros_like(ks)
    ks[:, :s] = k_b[:, :s]
    vs[:, :s] = v_b[:, :s]
    a = s + n_pages * w.N
    rest = T - a
    assert 0 <= rest <= w.N
    kr = np.zeros((w.H_kv, w.N, w.d), np.uint16)
    vr = np.zeros_like(kr)
    kr[:, :rest] = k_b[:, a:T]
    vr[:, :rest] = v_b[:, a:T]
    return oracle.decode_attn_f64(oc, qd_b, ks, vs, kp, vp, kr, vr, mask_b, s, n_pages, rest,
                                  sm_scale)


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def sm_scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))
