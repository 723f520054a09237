"""Pins of the oracle's float64 decode attention.

Eq. 1 (PN-Mix paper sec. 2) is plain GQA softmax attention; the cache of sec. 5 is FP16 sinks,
quantized pages and an FP16 residual buffer.  Pins: with no quantized pages the result is
torch's scaled_dot_product_attention in float64 over the fp16 tokens (a library routine); with
pages it equals the same routine over the densely dequantized cache; the query-to-KV head map
is floor(h' / n_g); and the attention over sinks alone carries no quantization error.
"""
import math

import numpy as np
import pytest
import torch

import synth


def _cache(orc, cfg, n_pages, res_len, sink_len, seed, max_pages=None):
    max_pages = max_pages or max(n_pages, 1)
    T = sink_len + n_pages * cfg.N + res_len
    sk = synth.pair_scales(cfg.H_kv, cfg.d // 2, 1.0, "cpu", "oracle-dec", seed, "k")
    sq = synth.pair_scales(cfg.H_q, cfg.d // 2, 1.0, "cpu", "oracle-dec", seed, "q")
    k = synth.rope_tokens(sk, 1, torch.arange(T), cfg.d, cfg.pairing, 1e4, "cpu", "oracle-dec",
                          seed, "k")[0].numpy()
    v = synth.values(1, cfg.H_kv, T, cfg.d, "cpu", "oracle-dec", seed)[0].numpy()
    q = synth.rope_tokens(sq, 1, torch.tensor([T]), cfg.d, cfg.pairing, 1e4, "cpu",
                          "oracle-dec", seed, "q")[0, :, 0].numpy()
    mask = np.zeros((cfg.H_kv, (cfg.d // 2 + 31) // 32), np.uint32)
    rng = np.random.default_rng(seed)
    for h in range(cfg.H_kv):
        for p in rng.choice(cfg.d // 2, cfg.n_hi_pairs, replace=False):
            mask[h, p // 32] |= np.uint32(1 << (int(p) % 32))
    k_sink = np.zeros((cfg.H_kv, cfg.N_s, cfg.d), np.float16)
    v_sink = np.zeros_like(k_sink)
    k_sink[:, :sink_len] = k[:, :sink_len]
    v_sink[:, :sink_len] = v[:, :sink_len]
    kp = np.zeros((cfg.H_kv, max_pages, orc.k_page_bytes(cfg)), np.uint8)
    vp = np.zeros((cfg.H_kv, max_pages, orc.v_page_bytes(cfg)), np.uint8)
    kdq = np.zeros((cfg.H_kv, T, cfg.d))
    vdq = np.zeros((cfg.H_kv, T, cfg.d))
    kdq[:, :sink_len] = k[:, :sink_len]
    vdq[:, :sink_len] = v[:, :sink_len]
    for h in range(cfg.H_kv):
        for p in range(n_pages):
            a = sink_len + p * cfg.N
            kp[h, p] = orc.quantize_k_page(cfg, k[h, a:a + cfg.N].view(np.uint16), mask[h])
            vp[h, p] = orc.quantize_v_page(cfg, v[h, a:a + cfg.N].view(np.uint16))
            kdq[h, a:a + cfg.N] = orc.dequant_k_page(cfg, kp[h, p], mask[h])
            vdq[h, a:a + cfg.N] = orc.dequant_v_page(cfg, vp[h, p])
    a = sink_len + n_pages * cfg.N
    k_res = np.zeros((cfg.H_kv, cfg.N, cfg.d), np.float16)
    v_res = np.zeros_like(k_res)
    k_res[:, :res_len] = k[:, a:a + res_len]
    v_res[:, :res_len] = v[:, a:a + res_len]
    kdq[:, a:] = k[:, a:]
    vdq[:, a:] = v[:, a:]
    return dict(q=q, k_sink=k_sink, v_sink=v_sink, k_pages=kp, v_pages=vp, k_res=k_res,
                v_res=v_res, mask=mask, kdq=kdq, vdq=vdq, k=k, v=v)


def _sdpa(cfg, q, K, V, scale):
    """torch SDPA in float64 with query heads mapped to KV heads by repeat_interleave."""
    qt = torch.from_numpy(q.astype(np.float64)).view(1, cfg.H_q, 1, cfg.d)
    Kt = torch.from_numpy(K).repeat_interleave(cfg.n_g, dim=0).unsqueeze(0)
    Vt = torch.from_numpy(V).repeat_interleave(cfg.n_g, dim=0).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt.contiguous(), Vt.contiguous(),
                                                         scale=scale)
    return o[0, :, 0].numpy()


@pytest.mark.parametrize("n_pages,res_len,sink_len", [(0, 57, 32), (0, 0, 32), (0, 128, 7),
                                                      (2, 96, 32), (3, 1, 32), (1, 128, 32)])
def test_decode_matches_sdpa(orc, n_pages, res_len, sink_len):
    cfg = orc.Cfg(H_q=8, H_kv=2, d=64, pairing=1, n_hi_pairs=16)
    c = _cache(orc, cfg, n_pages, res_len, sink_len, seed=n_pages * 7 + res_len)
    scale = float(np.float32(1.0 / math.sqrt(cfg.d)))
    out = orc.decode_attn_f64(cfg, c["q"], c["k_sink"], c["v_sink"], c["k_pages"], c["v_pages"],
                              c["k_res"], c["v_res"], c["mask"], sink_len, n_pages, res_len,
                              scale)
    ref = _sdpa(cfg, c["q"], c["kdq"], c["vdq"], scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    if n_pages == 0:
        # no quantized region: the fp16 cache is attended exactly (zero sink / residual error)
        exact = _sdpa(cfg, c["q"], c["k"].astype(np.float64), c["v"].astype(np.float64), scale)
        np.testing.assert_allclose(out, exact, rtol=0, atol=1e-12)


def test_gqa_head_map(orc):
    """Query head h' attends KV head floor(h'/n_g): moving a query head to another group
    changes its output to the other KV head's attention."""
    cfg = orc.Cfg(H_q=4, H_kv=2, d=32, pairing=0, n_hi_pairs=8)
    c = _cache(orc, cfg, 1, 40, 32, seed=3)
    scale = float(np.float32(1.0 / math.sqrt(cfg.d)))
    args = (c["k_sink"], c["v_sink"], c["k_pages"], c["v_pages"], c["k_res"], c["v_res"],
            c["mask"], 32, 1, 40, scale)
    out = orc.decode_attn_f64(cfg, c["q"], *args)
    q2 = c["q"][[2, 3, 0, 1]].copy()
    out2 = orc.decode_attn_f64(cfg, q2, *args)
    ref = _sdpa(cfg, q2, c["kdq"], c["vdq"], scale)
    np.testing.assert_allclose(out2, ref, atol=1e-12)
    assert not np.allclose(out2, out[[2, 3, 0, 1]], atol=1e-3)
