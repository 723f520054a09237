"""The fidelity analysis tool: metric helpers on the CPU, the packed-cache path on the GPU."""
import math

import numpy as np
import pytest
import torch

from decode_attention_pnmix_amd import fidelity as F


def test_mask_jaccard_counts_bits():
    a = torch.tensor([[[0b1011, 0]], [[0, 0]]], dtype=torch.int32)
    b = torch.tensor([[[0b0110, 0]], [[0, 0]]], dtype=torch.int32)
    j = F.mask_jaccard(a, b)
    assert j.shape == (2, 1)
    assert j[0, 0].item() == pytest.approx(1 / 4)   # {1} over {0, 1, 2, 3}
    assert j[1, 0].item() == 1.0                      # two empty masks
    hi = torch.tensor([[[0, -2**31]]], dtype=torch.int32)  # bit 63 of the pair mask
    assert F.mask_jaccard(hi, hi).item() == 1.0
    assert F.mask_jaccard(hi, torch.zeros_like(hi)).item() == 0.0


def test_reference_attention_matches_a_loop():
    g = torch.Generator().manual_seed(3)
    B, H_kv, ng, T, d = 2, 2, 3, 7, 8
    q = torch.randn(B, H_kv * ng, d, generator=g).half()
    k = torch.randn(B, H_kv, T, d, generator=g).half()
    v = torch.randn(B, H_kv, T, d, generator=g).half()
    sm = 1.0 / math.sqrt(d)
    out = F.reference_attention(q, k, v, sm).numpy()
    qn, kn, vn = q.double().numpy(), k.double().numpy(), v.double().numpy()
    for b in range(B):
        for h in range(H_kv * ng):
            lg = kn[b, h // ng] @ qn[b, h] * sm
            p = np.exp(lg - lg.max())
            p /= p.sum()
            assert np.abs(out[b, h] - p @ vn[b, h // ng]).max() < 1e-5


def test_output_errors():
    r = torch.tensor([[[1.0, 0.0], [0.0, 2.0]]])
    e = F.output_errors(r.clone(), r)
    assert e["mse"] == 0.0 and e["max_abs"] == 0.0 and e["rel_l2"] == 0.0
    assert e["cos_min"] == pytest.approx(1.0)
    o = torch.tensor([[[0.0, 1.0], [0.0, 2.0]]])
    e = F.output_errors(o, r)
    assert e["cos_min"] == pytest.approx(0.0) and e["cos_mean"] == pytest.approx(0.5)
    assert e["max_abs"] == 1.0 and e["mse"] == pytest.approx(0.5)


@pytest.mark.gpu
def test_load_context_equals_bulk_fill():
    import decode_attention_pnmix_amd as P
    import synth
    from _cases import cfgs, fill_cache_bulk, layer_inputs
    for w, T in ((synth.WORKLOADS["tiny"], 512),
                 (synth.Workload("ctx", 1, 3, 8, 2, 64, 1, 1e4, 64, 700, 0.5, 64, g_V=16), 700)):
        lc, _ = cfgs(w)
        qp, k, v, _ = layer_inputs(w, 1, w.B, T)
        ref = fill_cache_bulk(w, lc, qp, k, v, T)
        c = P.PNMixLayerCache(lc, w.B, ref.max_pages)
        c.load_context(qp, k, v)
        torch.cuda.synchronize()
        for name in ("mask", "lens", "k_sink", "v_sink", "k_res", "v_res", "k_pages", "v_pages"):
            assert torch.equal(getattr(c, name), getattr(ref, name)), (w.name, name)


@pytest.mark.gpu
def test_decode_fidelity_and_overlap():
    import decode_attention_pnmix_amd as P
    import synth
    from _cases import cfgs, layer_inputs
    w = synth.WORKLOADS["tiny"]
    lc, _ = cfgs(w)
    qp, k, v, qd = layer_inputs(w, 2, w.B, w.T)
    res = {}
    for r in (0.0, w.r, 1.0):
        c = P.make_cfg(w.H_q, w.H_kv, w.d, w.pairing, P.pnmix_hi_pairs(r, w.d), G=w.G,
                       b_V=w.b_V, g_V=w.g_V, N_s=w.N_s, N=w.N)
        res[r] = F.decode_fidelity(c, qp, k, v, qd)
        assert all(math.isfinite(x) for x in res[r].values())
    print({r: (round(e["rel_l2"], 4), round(e["cos_mean"], 4), round(e["cos_min"], 4))
           for r, e in res.items()})
    # more 3-bit key channels, less output error: all 1-bit > PN-Mix(r) > all 3-bit
    assert res[0.0]["rel_l2"] > res[w.r]["rel_l2"] > res[1.0]["rel_l2"]
    # a prompt's masks agree with themselves; the decode-time window gives a proper fraction
    j = F.saliency_overlap(lc, qp, k[:, :, :w.P], qp, k[:, :, :w.P])
    assert torch.all(j == 1.0)
    j = F.saliency_overlap(lc, qp, k[:, :, :w.P], qp, k[:, :, w.T - w.P:].contiguous())
    assert torch.all((j >= 0) & (j <= 1))
