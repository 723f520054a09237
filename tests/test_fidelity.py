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


def test_attention_kl_hand_computed():
    # p = softmax([0, 0]) = (1/2, 1/2), q = softmax([0, ln 3]) = (1/4, 3/4):
    # KL(p || q) = 1/2 ln 2 + 1/2 ln(2/3) = 1/2 ln(4/3)
    ref = torch.tensor([[0.0, 0.0]], dtype=torch.float64)
    lg = torch.tensor([[0.0, math.log(3.0)]], dtype=torch.float64)
    assert F.attention_kl(ref, lg).item() == pytest.approx(0.5 * math.log(4 / 3), rel=1e-12)
    assert F.attention_kl(lg, lg).item() == pytest.approx(0.0, abs=1e-15)
    # shifting all logits changes nothing
    assert F.attention_kl(ref + 7.0, lg - 2.0).item() == pytest.approx(0.5 * math.log(4 / 3))


def test_top_set_ties_go_to_the_lower_pair():
    s = torch.tensor([[1.0, 3.0, 3.0, 0.5], [2.0, 2.0, 2.0, 2.0]])
    t = F._top_set(s, 2)
    assert t.tolist() == [[False, True, True, False], [True, True, False, False]]


def test_decode_time_overlap_hand_computed():
    """d = 4 (2 RoPE pairs, split-half: pair 0 = channels (0, 2), pair 1 = (1, 3)), n_hi = 1, one
    KV head with two query heads, two decoding steps; the prefill mask keeps pair 0.  Every
    number below is worked by hand from the definition."""
    # query head 0: step 0 pair norms (1, 2); step 1 (1, 1)   [pair 0 = channels 0, 2]
    # query head 1: step 0 (5, 1);          step 1 (2, 1)
    # keys: step 0 pair norms (1, 1); step 1 (3, 1)
    def row(n0, n1):  # channels (c0 of pair 0, c0 of pair 1, c1 of pair 0, c1 of pair 1)
        return [n0, n1, 0.0, 0.0]
    q = torch.tensor([[[row(1, 2), row(1, 1)], [row(5, 1), row(2, 1)]]], dtype=torch.float64)
    k = torch.tensor([[[row(1, 1), row(3, 1)]]], dtype=torch.float64)
    mask = torch.tensor([[[0b01]]], dtype=torch.int32)
    # eligible (t, s): (0, 0), (1, 0), (1, 1), each for both query heads = 6 pairs
    # products per pair (pair0, pair1):
    #   head 0: (0,0): (1, 2) -> top pair 1, miss; (1,0): (1, 1) tie -> pair 0, hit;
    #           (1,1): (3, 1) -> pair 0, hit
    #   head 1: (0,0): (5, 1) hit; (1,0): (2, 1) hit; (1,1): (6, 1) hit
    res = F.decode_time_overlap(mask, q, k, pairing=1, n_hi=1, score="pair_norm", bins=2)
    assert res["pairs"] == 6
    assert res["overlap"] == pytest.approx(5 / 6)
    assert res["jaccard"] == pytest.approx((5 * 1 + 1 * 0) / 6)   # a miss has |A | M| = 2
    # step 0 bin: head 0 miss, head 1 hit -> 1/2; step 1 bin: all 4 hits -> 1
    assert res["overlap_bins"] == pytest.approx([0.5, 1.0])
    assert res["overlap_spread"] == pytest.approx(0.5)
    # |<q_i, k_i>| uses the angle too: keys orthogonal to the query in pair 0 lose it
    k2 = torch.tensor([[[[0.0, 1.0, 1.0, 0.0], [0.0, 1.0, 3.0, 0.0]]]], dtype=torch.float64)
    res2 = F.decode_time_overlap(mask, q, k2, pairing=1, n_hi=1, score="abs_dot")
    # pair 0 dot: q has only channel 0, keys only channel 2 -> 0; pair 1 dot = q1 k1 > 0 -> miss
    assert res2["overlap"] == 0.0


@pytest.mark.gpu
def test_attention_kl_overlap_and_reselection_on_the_gpu():
    import decode_attention_pnmix_amd as P
    import synth
    from _cases import cfgs, layer_inputs
    w = synth.Workload("fid", 1, 2, 8, 2, 64, 1, 1e4, 141, 32 + 4 * 128 + 40, 0.5, 64)
    lc, _ = cfgs(w)
    T = w.T
    qp, k, v, qd = layer_inputs(w, 4, w.B, T)
    sq = synth.pair_scales(w.H_q, w.d // 2, 1.0, "cuda", w.name, 4, "q")
    q_all = synth.rope_tokens(sq, w.B, torch.arange(T, device="cuda"), w.d, w.pairing, 1e4,
                              "cuda", w.name, 4, "qall")
    q_all[:, :, :w.P] = qp
    q_all[:, :, T - 1] = qd
    kls = {}
    for r in (0.0, 0.5, 1.0):
        c = P.make_cfg(w.H_q, w.H_kv, w.d, w.pairing, P.pnmix_hi_pairs(r, w.d), G=w.G,
                       b_V=w.b_V, g_V=w.g_V, N_s=w.N_s, N=w.N)
        cache = P.PNMixLayerCache(c, w.B, (T - w.N_s) // w.N)
        cache.load_context(qp, k, v)
        res = F.packed_vs_fp16(cache, qd, k, v)
        kls[r] = res["attn_kl_mean"]
        assert res["max_sink_key_error"] == 0.0
        # the analysis logits reproduce the decode kernel: softmax(logits) . V^ (values
        # dequantized by the library) against pnmix_decode_attn
        lg = F.attention_logits_packed(cache, qd)
        n_p = cache.n_pages
        vx = P.pnmix_dequant_v_pages(c, cache.v_pages[:, :n_p].reshape(-1, cache.v_pages.shape[-1])
                                     .contiguous())
        vx = vx.view(w.B, n_p, w.H_kv, w.N, w.d).permute(0, 2, 1, 3, 4).reshape(w.B, w.H_kv, -1, w.d)
        vall = torch.cat([cache.v_sink[:, :, :cache.sink_len].double(), vx.double(),
                          cache.v_res[:, :, :cache.res_len].double()], 2)
        p = torch.softmax(lg, -1).view(w.B, w.H_kv, w.H_q // w.H_kv, -1)
        ref = torch.matmul(p, vall).view(w.B, w.H_q, w.d)
        out = cache.attend(qd)
        assert (out.double() - ref).abs().max().item() <= 2e-3
        if r == 0.5:
            abl = F.reselection_ablation(c, q_all, k, w.P)
            assert abl["pages"] == n_p and abl["index_bytes_per_page_and_kv_head"] == 4
            # the fixed arm is this very cache
            assert abl["fixed"]["attn_kl_mean"] == pytest.approx(res["attn_kl_mean"], rel=1e-9)
            assert math.isfinite(abl["reselected"]["attn_kl_mean"])
            dt = F.decode_time_overlap(cache.mask, q_all[:, :, w.P:].contiguous(),
                                       k[:, :, w.P:].contiguous(), w.pairing, c.n_hi_pairs)
            assert 0.0 <= dt["overlap"] <= 1.0 and dt["pairs"] > 0
    assert kls[0.0] > kls[0.5] > kls[1.0] >= 0.0
