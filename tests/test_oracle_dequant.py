"""Pins of the oracle's page dequantizers against the inputs they came from.

The decode pin of the oracle (softmax attention over the cache) reads packed pages through
``dequant_k_page`` / ``dequant_v_page``, so these are checked here against what Eq. 2 and
Eq. 7 fix about the reconstruction of the ORIGINAL values (PN-Mix paper sec. 2, Eq. 2:
x^ = s q + z; reproduction notes "PN-Mix: Key-Cache Precision Allocation from RoPE Channel-Pair
Norms", Core equations: Eq. 7 levels of 1-bit groups at the bin midpoints, constant groups
stored with zero scale and the original offset), never against the dequantizer's own formula:
* every element lies within half a quantization step of its input, plus the fp16 rounding of
  the stored scale and offset: |x^ - x| <= s/2 + L * |h(s) - s| with s = (max - min) / L of the
  input group, computed here from the input in float64;
* a constant group reconstructs its input exactly;
* a 1-bit group (Eq. 7) reconstructs only to h((3 min + max)/4) and that level plus
  h((max - min)/2), the closed forms evaluated here in float64 from the input.
The pages are built so that neighbouring groups have very different offsets (each key token
group and each value channel group is shifted by its own constant), so reading the scale or
offset of the wrong group, or swapping scale and offset, breaks the first bound.
"""
import numpy as np
import pytest
import torch

import synth


def _h(x):
    """float64 -> fp16 (round half to even) -> float64"""
    return float(np.float16(x))


def _salient(cfg, orc, mask):
    s = np.zeros(cfg.d, bool)
    for i in range(cfg.d // 2):
        if (int(mask[i // 32]) >> (i % 32)) & 1:
            c0, c1 = orc.pair_channels(cfg, i)
            s[c0] = s[c1] = True
    return s


def _check_group(v, xh, L):
    """v: input group (float64), xh: its reconstruction, L = 2^b - 1 levels."""
    mn, mx = v.min() + 0.0, v.max() + 0.0
    if mx == mn:
        assert np.array_equal(xh, v), "a constant group reconstructs exactly"
        return
    if L == 1:
        lo, step = _h((3 * mn + mx) / 4), _h((mx - mn) / 2)
        assert np.all((xh == lo) | (xh == lo + step)), "Eq. 7 levels"
        bound = (mx - mn) / 4 * (1 + 1e-6) + 2 ** -11 * (abs(lo) + step) + 2 ** -23
    else:
        s = (mx - mn) / L
        bound = s / 2 * (1 + 1e-6) + L * 2 ** -11 * s + 2 ** -24
    err = np.abs(xh - v)
    assert err.max() <= bound, (err.max(), bound)


@pytest.mark.parametrize("G,bH,bL,r,pairing", [(128, 3, 1, 0.5, 1), (64, 3, 1, 0.4, 1),
                                                (32, 3, 1, 0.5, 0), (64, 4, 2, 0.3, 1),
                                                (32, 2, 1, 0.6, 0), (128, 4, 3, 0.2, 1)])
def test_dequant_k_page_against_inputs(orc, G, bH, bL, r, pairing):
    d = 64
    cfg = orc.Cfg(H_q=1, H_kv=1, d=d, pairing=pairing, n_hi_pairs=orc.hi_pairs(r, d), G=G,
                  b_H=bH, b_L=bL)
    sc = synth.pair_scales(1, d // 2, 1.0, "cpu", "dequant-k", G, bH)
    x = synth.rope_tokens(sc, 1, torch.arange(128) + 77, d, pairing, 1e4, "cpu", "dequant-k",
                          G, bH)[0, 0].float()
    x += (torch.arange(128) // G).float().view(-1, 1) * 24.0  # each token group its own offset
    x[:, 3] = 0.75  # a constant channel
    x = x.to(torch.float16).numpy()
    rng = np.random.default_rng(G + bH)
    mask = np.zeros((d // 2 + 31) // 32, np.uint32)
    for p in rng.choice(d // 2, cfg.n_hi_pairs, replace=False):
        mask[p // 32] |= np.uint32(1 << (int(p) % 32))
    page = orc.quantize_k_page(cfg, x.view(np.uint16), mask)
    xh = orc.dequant_k_page(cfg, page, mask)
    sal = _salient(cfg, orc, mask)
    xf = x.astype(np.float64)
    for g in range(128 // G):
        for c in range(d):
            _check_group(xf[g * G:(g + 1) * G, c], xh[g * G:(g + 1) * G, c],
                         2 ** (bH if sal[c] else bL) - 1)


@pytest.mark.parametrize("g_V,bV", [(16, 2), (32, 2), (64, 2), (32, 4), (16, 1), (64, 4)])
def test_dequant_v_page_against_inputs(orc, g_V, bV):
    d = 128
    cfg = orc.Cfg(H_q=1, H_kv=1, d=d, pairing=1, n_hi_pairs=16, g_V=g_V, b_V=bV)
    g = torch.Generator().manual_seed(g_V + bV)
    x = torch.randn(128, d, generator=g)
    x += (torch.arange(d) // g_V).float().view(1, -1) * 20.0  # each channel group its own offset
    x[5, g_V:2 * g_V] = -2.25  # a constant group
    x = x.to(torch.float16).numpy()
    page = orc.quantize_v_page(cfg, x.view(np.uint16))
    xh = orc.dequant_v_page(cfg, page)
    xf = x.astype(np.float64)
    for t in range(128):
        for gi in range(d // g_V):
            sl = slice(gi * g_V, (gi + 1) * g_V)
            _check_group(xf[t, sl], xh[t, sl], 2 ** bV - 1)
