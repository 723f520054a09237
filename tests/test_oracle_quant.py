"""Pins of the oracle's key and value page quantizers and their packing.

Eq. 2 (PN-Mix paper sec. 2; reproduction notes, Core equations): asymmetric b-bit min-max
group quantization, x^ = s q + z.  Eq. 7: a 1-bit group's two levels move to the bin
midpoints (3 min + max)/4 and (min + 3 max)/4.  Constant groups store zero scale and the
original offset.  Packing: the kernel-implementation appendix of the paper.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packing_example.json")


def _hexbytes(rows):
    return np.array([int(b, 16) for r in rows for b in r.split()], np.uint8)


def _hexf16(rows):
    return np.array([int(b, 16) for r in rows for b in r.split()], np.uint16)


def test_golden_k_page(orc):
    g = json.load(open(GOLDEN))
    cfg = orc.Cfg(**g["cfg"])
    kv = g["k"]
    src = np.zeros((cfg.N, cfg.d), np.float16)
    for ch, vals in kv["values"].items():
        src[:, int(ch)] = vals
    mask = np.array(kv["mask_row"], np.uint32)
    page = orc.quantize_k_page(cfg, src.view(np.uint16), mask)
    lo = _hexbytes(kv["lo_hex"])
    hi = _hexbytes(kv["hi_hex"])
    S = _hexf16(kv["S_f16_hex"]).view(np.uint8)
    Z = _hexf16(kv["Z_f16_hex"]).view(np.uint8)
    assert np.array_equal(page, np.concatenate([lo, hi, S, Z]))


def test_golden_v_page(orc):
    g = json.load(open(GOLDEN))
    cfg = orc.Cfg(**g["cfg"])
    vv = g["v"]
    src = np.zeros((cfg.N, cfg.d), np.float16)
    for t in range(cfg.N):
        src[t, :4] = [0, 1, 2, 3]
        src[t, 4:] = [t / 2] * 4 if t % 2 == 0 else [-3, 3, -2, 2]
    page = orc.quantize_v_page(cfg, src.view(np.uint16))
    codes = _hexbytes(vv["codes_hex"])
    # S and Z are stored group-major: [d/g_V][N]
    S = np.zeros((2, cfg.N), np.uint16)
    Z = np.zeros((2, cfg.N), np.uint16)
    zeven = _hexf16(vv["Z_f16_hex_group1_even_tokens"])
    for t in range(cfg.N):
        S[:, t] = [0x3C00, 0x0000 if t % 2 == 0 else 0x4000]
        Z[:, t] = [0x0000, zeven[t // 2] if t % 2 == 0 else 0xC200]
    assert np.array_equal(page, np.concatenate([codes, S.reshape(-1).view(np.uint8),
                                                Z.reshape(-1).view(np.uint8)]))


@pytest.mark.parametrize("name", ["k_h4_l2", "k_h4_l3"])
def test_golden_k_page_general_widths(orc, name):
    kv = json.load(open(GOLDEN))["general_widths"][name]
    cfg = orc.Cfg(**kv["cfg"])
    src = np.zeros((cfg.N, cfg.d), np.float16)
    for ch, vals in kv["values"].items():
        src[:, int(ch)] = vals
    mask = np.array(kv["mask_row"], np.uint32)
    page = orc.quantize_k_page(cfg, src.view(np.uint16), mask)
    want = np.concatenate([_hexbytes(kv["lo_hex"]), _hexbytes(kv["hi_hex"]),
                           _hexf16(kv["S_f16_hex"]).view(np.uint8),
                           _hexf16(kv["Z_f16_hex"]).view(np.uint8)])
    assert page.size == orc.k_page_bytes(cfg) == want.size
    assert np.array_equal(page, want)
    codes, _, _ = orc.unpack_k_page(cfg, page, mask)
    assert np.array_equal(codes[:, 0], np.arange(16))  # channel 0 holds t, s = 1, z = 0


def _token_rows(spec, N):
    even, odd = (json.loads(spec[k]) for k in ("even", "odd"))
    return np.array([even if t % 2 == 0 else odd for t in range(N)], np.float16)


@pytest.mark.parametrize("name", ["v_b4", "v_b1"])
def test_golden_v_page_general_widths(orc, name):
    vv = json.load(open(GOLDEN))["general_widths"][name]
    cfg = orc.Cfg(**vv["cfg"])
    src = _token_rows(vv["token_values"], cfg.N)
    page = orc.quantize_v_page(cfg, src.view(np.uint16))
    ng = cfg.d // cfg.g_V
    S = np.zeros((ng, cfg.N), np.uint16)
    Z = np.zeros((ng, cfg.N), np.uint16)
    for t in range(cfg.N):
        par = "even" if t % 2 == 0 else "odd"
        S[:, t] = _hexf16([vv["S_f16_hex_per_token"][par]])
        Z[:, t] = _hexf16([vv["Z_f16_hex_per_token"][par]])
    want = np.concatenate([_hexbytes(vv["codes_hex"]), S.reshape(-1).view(np.uint8),
                           Z.reshape(-1).view(np.uint8)])
    assert page.size == orc.v_page_bytes(cfg) == want.size
    assert np.array_equal(page, want)


def test_v_page_b16_keeps_fp16_rows(orc):
    """b_V = 16 (the value cache the bit-width sweep keeps in full precision): the page is the
    token rows themselves and dequantizes to them exactly."""
    cfg = orc.Cfg(H_q=1, H_kv=1, d=32, pairing=0, n_hi_pairs=8, b_V=16)
    x = torch.randn(128, 32, generator=torch.Generator().manual_seed(2)).to(torch.float16).numpy()
    page = orc.quantize_v_page(cfg, x.view(np.uint16))
    assert page.size == 128 * 32 * 2 == orc.v_page_bytes(cfg)
    assert np.array_equal(page.view(np.uint16).reshape(128, 32), x.view(np.uint16))
    assert np.array_equal(orc.dequant_v_page(cfg, page), x.astype(np.float64))


def _page(cfg, seed, sigma_ln=1.0, const_channels=(), signed_zero=False):
    sc = synth.pair_scales(1, cfg.d // 2, sigma_ln, "cpu", "oracle-quant", seed)
    x = synth.rope_tokens(sc, 1, torch.arange(cfg.N) + 1000, cfg.d, cfg.pairing, 1e4, "cpu",
                          "oracle-quant", seed)[0, 0].numpy().copy()
    for c in const_channels:
        x[:, c] = x[0, c]
    if signed_zero:
        x[: cfg.N // 2, 0] = np.float16(-0.0)
        x[cfg.N // 2:, 0] = np.float16(0.0)
    return x


def _mask_for(cfg, pairs):
    words = np.zeros(orc_words(cfg), np.uint32)
    for p in pairs:
        words[p // 32] |= np.uint32(1 << (p % 32))
    return words


def orc_words(cfg):
    return (cfg.d // 2 + 31) // 32


def _salient(cfg, orc, mask):
    s = np.zeros(cfg.d, bool)
    for i in range(cfg.d // 2):
        if (int(mask[i // 32]) >> (i % 32)) & 1:
            c0, c1 = orc.pair_channels(cfg, i)
            s[c0] = s[c1] = True
    return s


@pytest.mark.parametrize("pairing,G,r,bH,bL", [
    (0, 128, 0.5, 3, 1), (1, 128, 0.5, 3, 1), (1, 64, 0.4, 3, 1), (1, 32, 0.25, 3, 1),
    (0, 128, 1.0, 3, 1), (1, 64, 0.0, 3, 1),
    # the bit-width sweep: b_H, b_L in {4, 3, 2, 1}, b_H >= b_L
    (1, 128, 0.3, 4, 2), (0, 64, 0.6, 4, 1), (1, 128, 0.5, 2, 1), (1, 64, 0.2, 4, 3),
    (0, 128, 0.5, 2, 2), (1, 128, 0.7, 4, 4), (1, 64, 0.5, 1, 1), (0, 32, 0.9, 3, 2)])
def test_k_page_levels(orc, pairing, G, r, bH, bL):
    d = 128
    cfg = orc.Cfg(H_q=1, H_kv=1, d=d, pairing=pairing, n_hi_pairs=orc.hi_pairs(r, d), G=G,
                  b_H=bH, b_L=bL)
    rng = np.random.default_rng(int(r * 100) + G)
    pairs = sorted(rng.choice(d // 2, cfg.n_hi_pairs, replace=False).tolist())
    mask = _mask_for(cfg, pairs)
    x = _page(cfg, seed=G + pairing, const_channels=(5, 77), signed_zero=True)
    page = orc.quantize_k_page(cfg, x.view(np.uint16), mask)
    assert page.size == (cfg.N * d * bL // 8 + cfg.N * cfg.n_sal * (bH - bL) // 8 +
                         4 * (cfg.N // G) * d)
    codes, S, Z = orc.unpack_k_page(cfg, page, mask)
    sal = _salient(cfg, orc, mask)
    assert sal.sum() == cfg.n_sal
    xf = x.astype(np.float64)
    n_eq7_exc = 0
    for g in range(cfg.N // G):
        blk = xf[g * G:(g + 1) * G]
        cb = codes[g * G:(g + 1) * G]
        for c in range(d):
            v = blk[:, c]
            mn, mx = v.min() + 0.0, v.max() + 0.0
            q = cb[:, c].astype(np.int64)
            Sg = float(np.uint16(S[g, c]).view(np.float16))
            Zg = float(np.uint16(Z[g, c]).view(np.float16))
            if mx == mn:
                # constant group: zero scale, original offset, exact reconstruction
                assert S[g, c] == 0 and np.all(q == 0)
                assert Zg == mn and np.all(Sg * q + Zg == v)
                continue
            L = 2 ** (bH if sal[c] else bL) - 1
            assert q.max() <= L
            levels = mn + np.arange(L + 1) * (mx - mn) / L
            # Eq. 2: the code is the nearest of the 2^b levels (fp64 reference levels); a
            # different choice is allowed only where two levels are within fp32 rounding of a tie
            dist = np.abs(v[:, None] - levels[None, :])
            best = dist.argmin(axis=1)
            amb = np.abs(dist[np.arange(len(v)), best] - dist[np.arange(len(v)), q]) <= \
                4e-7 * (mx - mn)
            assert np.all((q == best) | amb)
            # exact ties go to the even level
            tie = np.isclose(dist[np.arange(len(v)), q], (mx - mn) / L / 2, rtol=0, atol=0)
            assert np.all(q[tie] % 2 == 0)
            s32 = np.float32((np.float32(mx) - np.float32(mn)) / np.float32(L))
            assert np.all(np.abs(v - (float(s32) * q + mn)) <= float(s32) / 2 * (1 + 1e-6))
            if L == 1:
                # Eq. 7 closed form: levels (3 mn + mx)/4 and (mn + 3 mx)/4
                z7, s7 = (3 * mn + mx) / 4, (mx - mn) / 2
                if np.float16(z7) != np.float16(Zg) or np.float16(s7) != np.float16(Sg):
                    n_eq7_exc += 1
                assert abs(Zg - z7) <= 2 ** -10 * abs(z7) + 2 ** -24
                assert abs(Sg - s7) <= 2 ** -10 * abs(s7)
                assert abs((Zg + Sg) - (mn + 3 * mx) / 4) <= 2 ** -9 * (abs(mn) + abs(mx)) + 2 ** -23
                # codes of Eq. 2 with s = mx - mn: 1 exactly above the midpoint
                mid = (mn + mx) / 2
                assert np.all((q == 1) == (v > mid))
            else:
                assert float(np.float16(s32)) == Sg and Zg == mn
    assert n_eq7_exc == 0


def test_eq7_fp32_metadata_exact(orc):
    """With fp32 metadata the 1-bit levels equal the float64 closed forms exactly whenever those
    are representable in fp32 (always so for fp16 inputs of moderate range)."""
    cfg = orc.Cfg(H_q=1, H_kv=1, d=32, pairing=0, n_hi_pairs=0, G=128)
    rng = np.random.default_rng(3)
    for _ in range(200):
        v = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float16)
        mn, mx = np.float32(v.min()), np.float32(v.max())
        z7 = np.float32((np.float32(3.0) * mn + mx) * np.float32(0.25))
        s7 = np.float32((mx - mn) * np.float32(0.5))
        assert float(z7) == (3 * float(mn) + float(mx)) / 4
        assert float(z7) + float(s7) == (float(mn) + 3 * float(mx)) / 4
        src = np.zeros((128, 32), np.float16)
        src[:, 0] = v
        page = orc.quantize_k_page(cfg, src.view(np.uint16), np.zeros(1, np.uint32))
        _, S, Z = orc.unpack_k_page(cfg, page, np.zeros(1, np.uint32))
        assert S[0, 0] == np.float16(s7).view(np.uint16)
        assert Z[0, 0] == np.float16(z7).view(np.uint16)


def test_r1_is_uniform_3bit_and_r0_is_all_1bit(orc):
    d = 64
    x = _page(orc.Cfg(1, 1, d, 1, 0), seed=21)
    full = orc.Cfg(H_q=1, H_kv=1, d=d, pairing=1, n_hi_pairs=d // 2)
    none = orc.Cfg(H_q=1, H_kv=1, d=d, pairing=1, n_hi_pairs=0)
    pf = orc.quantize_k_page(full, x.view(np.uint16), np.array([0xFFFFFFFF], np.uint32))
    pn = orc.quantize_k_page(none, x.view(np.uint16), np.array([0], np.uint32))
    assert pn.size == 128 * d // 8 + 4 * d  # empty hi plane
    cf, Sf, Zf = orc.unpack_k_page(full, pf, np.array([0xFFFFFFFF], np.uint32))
    cn, Sn, Zn = orc.unpack_k_page(none, pn, np.array([0], np.uint32))
    xf = x.astype(np.float64)
    mn, mx = xf.min(0), xf.max(0)
    # r = 1: per-channel uniform 3-bit min-max (KIVI-style) on every channel
    assert np.all(Zf[0] == mn.astype(np.float16).view(np.uint16))
    assert cf.max() == 7
    # r = 0: every channel 1-bit, codes are the midpoint threshold
    assert cn.max() == 1
    assert np.array_equal(cn.astype(bool), xf > (mn + mx) / 2)
    # the LSB plane of r = 0 is not the LSB plane of r = 1 (different bit widths)
    assert not np.array_equal(pf[: 128 * d // 8], pn[: 128 * d // 8])


def test_k_rejects_wrong_popcount(orc):
    cfg = orc.Cfg(H_q=1, H_kv=1, d=32, pairing=0, n_hi_pairs=4)
    x = np.zeros((128, 32), np.uint16)
    with pytest.raises(ValueError):
        orc.quantize_k_page(cfg, x, np.array([0b111], np.uint32))


@pytest.mark.parametrize("g_V,bV", [(32, 2), (16, 2), (32, 4), (16, 4), (64, 1), (128, 1)])
def test_v_page_levels(orc, g_V, bV):
    d = 128
    cfg = orc.Cfg(H_q=1, H_kv=1, d=d, pairing=1, n_hi_pairs=32, g_V=g_V, b_V=bV)
    L = 2 ** bV - 1
    g = torch.Generator().manual_seed(5 + bV)
    x = torch.randn(128, d, generator=g).to(torch.float16).numpy()
    x[3, :g_V] = 1.5  # a constant group
    page = orc.quantize_v_page(cfg, x.view(np.uint16))
    assert page.size == 128 * d * bV // 8 + 4 * 128 * (d // g_V)
    codes, S, Z = orc.unpack_v_page(cfg, page)
    xf = x.astype(np.float64)
    for t in range(128):
        for gi in range(d // g_V):
            v = xf[t, gi * g_V:(gi + 1) * g_V]
            q = codes[t, gi * g_V:(gi + 1) * g_V].astype(np.int64)
            mn, mx = v.min() + 0.0, v.max() + 0.0
            Sg = float(np.uint16(S[t, gi]).view(np.float16))
            Zg = float(np.uint16(Z[t, gi]).view(np.float16))
            if mn == mx:
                assert S[t, gi] == 0 and np.all(q == 0) and Zg == mn
                continue
            assert q.max() <= L
            levels = mn + np.arange(L + 1) * (mx - mn) / L
            dist = np.abs(v[:, None] - levels[None, :])
            best = dist.argmin(axis=1)
            amb = np.abs(dist[np.arange(g_V), best] - dist[np.arange(g_V), q]) <= 4e-7 * (mx - mn)
            assert np.all((q == best) | amb)
            s32 = (np.float32(mx) - np.float32(mn)) / np.float32(L)
            assert np.all(np.abs(v - (float(s32) * q + mn)) <= float(s32) / 2 * (1 + 1e-6))
            if L == 1:  # Eq. 7 metadata for a 1-bit value group
                assert Sg == float(np.float16((mx - mn) / 2))
                assert Zg == float(np.float16((3 * mn + mx) / 4))
                assert np.all((q == 1) == (v > (mn + mx) / 2))
            else:
                assert Zg == mn and Sg == float(np.float16(s32))


def test_page_sizes_and_printed_average_bits(orc):
    """Page sizes of the five workloads, and the average key bit-width the pages print for the
    two operating points (2.26 for r = 0.5, G = 128; 2.29 for r = 0.4, G = 64; Korean summary,
    "어떻게 쓰나"), recomputed from this layout's K page size at T_q = 32,768 (bit-width
    appendix): payload + fp16 scale/zero per page, plus N_s = 32 fp16 sink tokens, over
    (T_q + N_s) d key elements; the mask is metadata counted separately."""
    c1 = orc.Cfg(32, 8, 128, 1, orc.hi_pairs(0.5, 128), G=128)
    c2 = orc.Cfg(32, 8, 128, 1, orc.hi_pairs(0.4, 128), G=64)
    ct = orc.Cfg(4, 2, 32, 0, orc.hi_pairs(0.5, 32), G=128)
    assert (orc.k_page_bytes(c1), orc.v_page_bytes(c1)) == (4608, 6144)
    assert orc.k_page_bytes(c2) == 4672
    assert (orc.k_page_bytes(ct), orc.v_page_bytes(ct)) == (1152, 1536)
    Tq, Ns, d = 32768, 32, 128
    for cfg, printed in ((c1, "2.26"), (c2, "2.29")):
        bits = (orc.k_page_bytes(cfg) * 8 * (Tq // 128) + Ns * d * 16) / ((Tq + Ns) * d)
        assert f"{bits:.2f}" == printed, bits
