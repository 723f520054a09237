"""GPU parity over the bit-width sweep and the generic decode kernel, through the C ABI.

The PN-Mix paper's Table 14 / Figure 3 sweep b_H, b_L in {4, 3, 2, 1} (b_H >= b_L) with the
value cache kept at b_V = 16; the library also packs b_V in {1, 2, 4}.  Page quantization and
packing are bit-exact against the oracle at every width; the dequantized pages of the analysis
entry points equal the oracle's reconstruction rounded to fp32; decode attention on the generic
kernel (every setting but (3, 1, 2) with value groups of >= 32 channels, and (3, 1, 2) with
16-channel value groups) is within 2e-3 of the float64 oracle, and its paged and fused entry
points agree with the contiguous and the unfused ones bit for bit.
"""
import numpy as np
import pytest
import torch

import decode_attention_pnmix_amd as P
import oracle
import synth
from _cases import cfgs, fill_cache_bulk, layer_inputs, oracle_decode, say, sm_scale, u16

pytestmark = pytest.mark.gpu

ATOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    P.lib()


def _wl(name, d=128, H_q=16, H_kv=2, r=0.5, G=128, g_V=32, bH=3, bL=1, bV=2, B=2,
        T=32 + 3 * 128 + 50, pairing=1):
    return synth.Workload(name, 1, B, H_q, H_kv, d, pairing, 1e4, 64, T, r, G, b_V=bV, g_V=g_V,
                          b_H=bH, b_L=bL)


# (b_H, b_L, b_V, G, g_V, d): the sweep's widths, each G, each value width, both head dims
WIDTHS = [(4, 2, 16, 64, 32, 128), (4, 1, 2, 128, 32, 128), (2, 1, 4, 64, 32, 128),
          (4, 3, 1, 32, 64, 128), (2, 2, 16, 128, 32, 64), (1, 1, 4, 128, 16, 64),
          (4, 4, 2, 64, 32, 32), (3, 2, 1, 128, 32, 128), (3, 1, 16, 128, 32, 128),
          (3, 1, 2, 64, 16, 64)]


def _pages(lc, d, n, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, 128, d, generator=g) * torch.exp(torch.randn(n, 1, d, generator=g) * 1.5)
    x[0, :, 3] = 0.5            # a constant channel
    x[1, :, :] = 2.0            # a constant page
    x[2, 5, :] = -0.0
    xh = x.to(torch.float16)
    bits = torch.randint(0, 1 << 16, (2, 128, d), generator=g, dtype=torch.int32)
    bits = torch.where((bits & 0x7C00) == 0x7C00, bits & 0x83FF, bits)
    xh[3:5] = bits.to(torch.int16).view(torch.float16)
    words = P.pnmix_mask_words(lc)
    masks = torch.zeros(n, words, dtype=torch.int64)
    for i in range(n):
        for p in torch.randperm(d // 2, generator=g)[:lc.n_hi_pairs].tolist():
            masks[i, p // 32] |= 1 << (p % 32)
    return xh.cuda().contiguous(), masks.to(torch.int32).cuda().contiguous()


@pytest.mark.parametrize("bH,bL,bV,G,g_V,d", WIDTHS)
def test_quant_and_dequant_general_widths(bH, bL, bV, G, g_V, d):
    w = _wl("widths", d=d, G=G, g_V=g_V, bH=bH, bL=bL, bV=bV, r=0.4)
    lc, oc = cfgs(w)
    say(f"[quant-widths] b_H={bH} b_L={bL} b_V={bV} G={G} g_V={g_V} d={d}")
    n = 24
    src, masks = _pages(lc, d, n, seed=bH * 100 + bL * 10 + bV)
    kpb, vpb = P.pnmix_k_page_bytes(lc), P.pnmix_v_page_bytes(lc)
    assert (kpb, vpb) == (oracle.k_page_bytes(oc), oracle.v_page_bytes(oc))
    kd = torch.zeros(n, kpb, dtype=torch.uint8, device="cuda")
    vd = torch.zeros(n, vpb, dtype=torch.uint8, device="cuda")
    srcs = [src.data_ptr() + i * 128 * d * 2 for i in range(n)]
    P.pnmix_quantize_k_page(lc, P.page_jobs(srcs, d, [kd.data_ptr() + i * kpb for i in range(n)],
                                            range(n), "cuda"), masks)
    P.pnmix_quantize_v_page(lc, P.page_jobs(srcs, d, [vd.data_ptr() + i * vpb for i in range(n)],
                                            range(n), "cuda"))
    kx = P.pnmix_dequant_k_pages(lc, kd, masks)
    vx = P.pnmix_dequant_v_pages(lc, vd)
    torch.cuda.synchronize()
    sh, mh = u16(src), masks.cpu().numpy().view(np.uint32)
    kg, vg, kxg, vxg = kd.cpu().numpy(), vd.cpu().numpy(), kx.cpu().numpy(), vx.cpu().numpy()
    for i in range(n):
        ko = oracle.quantize_k_page(oc, sh[i], mh[i])
        vo = oracle.quantize_v_page(oc, sh[i])
        assert np.array_equal(kg[i], ko), f"K page {i}"
        assert np.array_equal(vg[i], vo), f"V page {i}"
        # reconstruction: the oracle's float64 S q + Z rounded to fp32 (one rounding on both
        # sides; pages 3-4 hold random bit patterns whose S q + Z can need more than 53 bits)
        kr = oracle.dequant_k_page(oc, ko, mh[i]).astype(np.float32)
        vr = oracle.dequant_v_page(oc, vo).astype(np.float32)
        if i in (3, 4):
            assert np.allclose(kxg[i], kr, rtol=2 ** -23, atol=0, equal_nan=True)
            assert np.allclose(vxg[i], vr, rtol=2 ** -23, atol=0, equal_nan=True)
        else:
            assert np.array_equal(kxg[i], kr), f"K dequant page {i}"
            assert np.array_equal(vxg[i], vr), f"V dequant page {i}"


DEC_CASES = [
    # id, bH, bL, bV, G, g_V, d, H_q, H_kv, B
    ("h4l2-v16", 4, 2, 16, 64, 32, 128, 16, 2, 2),
    ("h4l1-v2", 4, 1, 2, 128, 32, 128, 8, 2, 3),
    ("h2l1-v4-d64", 2, 1, 4, 64, 32, 64, 12, 2, 2),
    ("h4l3-v1", 4, 3, 1, 32, 64, 128, 4, 4, 2),
    ("h2l2-v16-d32", 2, 2, 16, 128, 32, 32, 4, 2, 2),
    ("h1l1-v4", 1, 1, 4, 128, 16, 64, 32, 2, 2),
    ("h3l1-v16", 3, 1, 16, 128, 32, 128, 8, 2, 40),
    ("h3l1-v2-gV16", 3, 1, 2, 64, 16, 64, 8, 2, 2),
    ("h3l1-v2-gV16-d32", 3, 1, 2, 128, 16, 32, 6, 2, 1),
    # (r, pairing) other than (0.5, split-half): upper-plane rows of 38 bytes (2-byte aligned),
    # no upper plane, every channel salient; 4-bit and 3-bit LSB planes; adjacent pairs
    ("h4l1-v2-r03", 4, 1, 2, 64, 32, 128, 16, 2, 2, 0.3, 1),
    ("h2l1-v16-r0", 2, 1, 16, 128, 64, 128, 8, 2, 2, 0.0, 1),
    ("h3l2-v4-r1-adj", 3, 2, 4, 64, 32, 64, 16, 4, 2, 1.0, 0),
    ("h4l4-v2-d32", 4, 4, 2, 64, 16, 32, 8, 1, 3, 0.5, 1),
    ("h3l3-v1-adj", 3, 3, 1, 128, 32, 128, 4, 2, 2, 0.5, 0),
    ("h4l3-v16-r07", 4, 3, 16, 64, 32, 128, 24, 4, 2, 0.7, 1),
    # 16 query heads per KV head with 32-token groups and fp16 values: the tables exceed 64 KiB
    # of LDS and the vector-ALU kernel serves the call
    ("h4l1-v16-ng16-G32", 4, 1, 16, 32, 32, 128, 32, 2, 1),
]


@pytest.mark.parametrize("case", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_generic_decode(case):
    name, bH, bL, bV, G, g_V, d, H_q, H_kv, B = case[:10]
    r, pairing = case[10:] if len(case) > 10 else (0.5, 1)
    T = 32 + 5 * 128 + 77
    w = _wl(name, d=d, H_q=H_q, H_kv=H_kv, r=r, G=G, g_V=g_V, bH=bH, bL=bL, bV=bV, B=B, T=T,
            pairing=pairing)
    lc, oc = cfgs(w)
    splits = P.pnmix_decode_splits(lc, B, w.n_pages)
    say(f"[decode-generic] {name} B={B} splits={splits} n_hi={lc.n_hi_pairs}")
    qp, k, v, qd = layer_inputs(w, 6, B, T)
    cache = fill_cache_bulk(w, lc, qp, k, v, T)
    out = cache.attend(qd)
    torch.cuda.synchronize()
    out_h = out.cpu().numpy()
    for b in sorted({0, B - 1}):
        ref = oracle_decode(w, oc, u16(qp[b]), u16(k[b]), u16(v[b]), u16(qd[b]), T,
                            sm_scale(d))
        err = np.abs(out_h[b] - ref).max()
        say(f"   b={b} max|err|={err:.3e}")
        assert err <= ATOL, (name, b, err)


def test_generic_decode_paged_and_fused():
    """The generic kernel behind the paged entry point (shuffled pool, junk table entries) and
    the fused step: equal to the contiguous call and to append-then-attend, bit for bit."""
    w = _wl("generic-paged", bH=4, bL=2, bV=16, G=64, B=3, T=32 + 4 * 128 + 9)
    lc, _ = cfgs(w)
    T = w.T
    qp, k, v, qd = layer_inputs(w, 8, w.B, T)
    n_pages = (T - w.N_s) // w.N
    c = fill_cache_bulk(w, lc, qp, k, v, T, max_pages=n_pages + 2)
    out_c = c.attend(qd)
    H, mp = w.H_kv, c.max_pages
    n_blocks = w.B * mp + 5
    gen = torch.Generator().manual_seed(3)
    perm = torch.randperm(n_blocks, generator=gen)[:w.B * mp].reshape(w.B, mp)
    kpb, vpb = P.pnmix_k_page_bytes(lc), P.pnmix_v_page_bytes(lc)
    k_pool = torch.randint(0, 256, (n_blocks, H, kpb), dtype=torch.uint8, generator=gen).cuda()
    v_pool = torch.randint(0, 256, (n_blocks, H, vpb), dtype=torch.uint8, generator=gen).cuda()
    idx = perm[:, :n_pages].reshape(-1).cuda()
    k_pool[idx] = c.k_pages[:, :n_pages].reshape(-1, H, kpb)
    v_pool[idx] = c.v_pages[:, :n_pages].reshape(-1, H, vpb)
    table = perm.to(torch.int32).clone()
    table[:, n_pages:] = -3
    out_p = P.pnmix_decode_attn_paged(lc, qd, c.k_sink, c.v_sink, k_pool, v_pool, table.cuda(),
                                      c.k_res, c.v_res, c.lens, c.mask, c.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_c)
    # fused step from a short prompt across a page flush
    wf = synth.Workload("generic-fused", 1, 2, 8, 2, 64, 1, 1e4, 5, 205, 0.5, 64, b_V=4,
                        g_V=32, b_H=2, b_L=1)
    lf, _ = cfgs(wf)
    qp, k, v, _ = layer_inputs(wf, 1, wf.B, wf.T)
    sq = synth.pair_scales(wf.H_q, wf.d // 2, 1.0, "cuda", wf.name, 1, "q")
    mpf = (wf.T - wf.N_s) // wf.N + 1
    c1 = P.PNMixLayerCache(lf, wf.B, mpf)
    c2 = P.PNMixLayerCache(lf, wf.B, mpf)
    for cc in (c1, c2):
        cc.prefill(qp, k[:, :, :wf.P].contiguous(), v[:, :, :wf.P].contiguous())
    for t in range(wf.P, wf.T):
        qt = synth.rope_tokens(sq, wf.B, torch.tensor([t], device="cuda"), wf.d, wf.pairing,
                               1e4, "cuda", wf.name, 1, "qstep", t)[:, :, 0].contiguous()
        kt, vt = k[:, :, t].contiguous(), v[:, :, t].contiguous()
        o1 = c1.step(qt, kt, vt)
        c2.append(kt, vt)
        o2 = c2.attend(qt)
        c2.flush()
        assert torch.equal(o1, o2), t
    torch.cuda.synchronize()
    assert c1.n_pages == 1
    for nm in ("lens", "k_sink", "v_sink", "k_res", "v_res", "k_pages", "v_pages"):
        assert torch.equal(getattr(c1, nm), getattr(c2, nm)), nm
