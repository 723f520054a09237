"""Pins of the oracle's Eq. 6 prefill score and pair mask.

Eq. 6 (reproduction notes, Core equations): sigma_{h,i} is the GQA-averaged mean query pair
norm times the mean key pair norm over the prefill tokens; the top floor(r d/2) pairs of each
KV head go into a fixed mask.  The pins below are the full-grid joint identity (the mean over
all (t, s) of the product of norms equals the product of the means), the causal joint score
the separable form approximates (Korean summary page), rotation invariance (RoPE rotates each
pair, so scoring before or after RoPE gives the same mask only under the right pairing),
special cases and a brute-force sort of the selection.
"""
import numpy as np
import pytest
import scipy.stats
import torch

import synth


def _inputs(cfg, P, sigma_ln=1.0, base=1e4, seed=0, pre_rope=False):
    sq = synth.pair_scales(cfg.H_q, cfg.d // 2, sigma_ln, "cpu", "oracle-score", seed, "q")
    sk = synth.pair_scales(cfg.H_kv, cfg.d // 2, sigma_ln, "cpu", "oracle-score", seed, "k")
    pos = torch.zeros(P) if pre_rope else torch.arange(P)
    q = synth.rope_tokens(sq, 1, pos, cfg.d, cfg.pairing, base, "cpu", "oracle-score", seed, "q")
    k = synth.rope_tokens(sk, 1, pos, cfg.d, cfg.pairing, base, "cpu", "oracle-score", seed, "k")
    return q[0].numpy().view(np.uint16), k[0].numpy().view(np.uint16)


def _norms64(orc, cfg, x):
    """float64 pair norms [H][P][d/2] from the channel pairing."""
    xf = orc.h2f(x).astype(np.float64)
    out = np.empty(xf.shape[:2] + (cfg.d // 2,))
    for i in range(cfg.d // 2):
        c0, c1 = orc.pair_channels(cfg, i)
        out[..., i] = np.hypot(xf[..., c0], xf[..., c1])
    return out


@pytest.mark.parametrize("pairing", [0, 1])
@pytest.mark.parametrize("ng", [1, 2, 4])
def test_sigma_equals_full_grid_joint_mean(orc, pairing, ng):
    cfg = orc.Cfg(H_q=2 * ng, H_kv=2, d=32, pairing=pairing, n_hi_pairs=8)
    P = 150  # three 64-token chunks, the last one ragged
    q, k = _inputs(cfg, P, seed=ng + 10 * pairing)
    qm, km, sigma, mask = orc.score_prefill(cfg, q, k)
    qn, kn = _norms64(orc, cfg, q), _norms64(orc, cfg, k)
    for h in range(cfg.H_kv):
        grid = np.zeros(cfg.d // 2)
        for hq in range(h * ng, (h + 1) * ng):
            # mean over every (t, s) of ||q_t|| ||k_s||, an O(P^2) sum
            grid += (qn[hq][:, None, :] * kn[h][None, :, :]).mean(axis=(0, 1))
        grid /= ng
        np.testing.assert_allclose(sigma[h], grid, rtol=2e-6)
    np.testing.assert_allclose(qm, qn.mean(axis=1), rtol=1e-6)
    np.testing.assert_allclose(km, kn.mean(axis=1), rtol=1e-6)


def test_separable_score_tracks_causal_joint_score(orc):
    cfg = orc.Cfg(H_q=4, H_kv=2, d=32, pairing=0, n_hi_pairs=8)
    P = 48
    q, k = _inputs(cfg, P, seed=3)
    _, _, sigma, mask = orc.score_prefill(cfg, q, k)
    joint = orc.joint_causal_score(cfg, q, k)
    for h in range(cfg.H_kv):
        rho = scipy.stats.spearmanr(sigma[h], joint[h]).statistic
        assert rho >= 0.9, rho
        top_sep = set(np.argsort(-sigma[h], kind="stable")[: cfg.n_hi_pairs])
        top_joint = set(np.argsort(-joint[h], kind="stable")[: cfg.n_hi_pairs])
        assert len(top_sep & top_joint) / cfg.n_hi_pairs >= 0.8


@pytest.mark.parametrize("pairing", [0, 1])
def test_mask_invariant_to_rope_rotation(orc, pairing):
    """Pair norms are rotation invariant, so the mask of pre-RoPE tokens (position 0) and of the
    same draws rotated to positions 0..P-1 agree wherever the sigma gap at the cut is clear."""
    cfg = orc.Cfg(H_q=8, H_kv=2, d=64, pairing=pairing, n_hi_pairs=16)
    P = 100
    q0, k0 = _inputs(cfg, P, seed=5, pre_rope=True)
    q1, k1 = _inputs(cfg, P, seed=5, pre_rope=False)
    _, _, s0, m0 = orc.score_prefill(cfg, q0, k0)
    _, _, s1, m1 = orc.score_prefill(cfg, q1, k1)
    for h in range(cfg.H_kv):
        srt = np.sort(s0[h])[::-1]
        gap = (srt[cfg.n_hi_pairs - 1] - srt[cfg.n_hi_pairs]) / srt[cfg.n_hi_pairs - 1]
        if gap > 1e-2:
            assert np.array_equal(m0[h], m1[h])
    # and a wrong pairing breaks the invariance on the same draws
    wrong = orc.Cfg(**{**cfg.__dict__, "pairing": 1 - pairing})
    _, _, w0, _ = orc.score_prefill(wrong, q0, k0)
    _, _, w1, _ = orc.score_prefill(wrong, q1, k1)
    assert not np.allclose(w0, w1, rtol=1e-2)


def _mask_pairs(mask_row, npairs):
    return [i for i in range(npairs) if (int(mask_row[i // 32]) >> (i % 32)) & 1]


@pytest.mark.parametrize("r", [0.0, 0.1, 0.4, 0.5, 0.9, 1.0])
def test_mask_is_top_floor_rd2_by_brute_force_sort(orc, r):
    d = 128
    cfg = orc.Cfg(H_q=8, H_kv=2, d=d, pairing=1, n_hi_pairs=orc.hi_pairs(r, d))
    assert cfg.n_hi_pairs == int(np.floor(r * d / 2 + 1e-9))
    q, k = _inputs(cfg, 70, seed=int(r * 10))
    _, _, sigma, mask = orc.score_prefill(cfg, q, k)
    for h in range(cfg.H_kv):
        # stable sort of (-sigma, index): descending sigma, ties to the lower pair index
        order = sorted(range(d // 2), key=lambda i: (-float(sigma[h][i]), i))
        assert _mask_pairs(mask[h], d // 2) == sorted(order[: cfg.n_hi_pairs])
        assert sum(bin(int(w)).count("1") for w in mask[h]) == cfg.n_hi_pairs


def test_mask_ties_go_to_lower_index(orc):
    cfg = orc.Cfg(H_q=1, H_kv=1, d=16, pairing=0, n_hi_pairs=3, g_V=8)
    P = 4
    # every pair has the same norm: all sigma equal, so pairs 0, 1, 2 are chosen
    q = np.full((1, P, 16), np.float16(1.0)).view(np.uint16)
    k = np.full((1, P, 16), np.float16(2.0)).view(np.uint16)
    _, _, sigma, mask = orc.score_prefill(cfg, q, k)
    assert np.all(sigma == sigma[0, 0])
    assert int(mask[0, 0]) == 0b111


def test_gqa_grouping_and_ng1(orc):
    cfg = orc.Cfg(H_q=4, H_kv=2, d=32, pairing=0, n_hi_pairs=4)
    q, k = _inputs(cfg, 40, seed=9)
    qm, km, sigma, _ = orc.score_prefill(cfg, q, k)
    # query heads (0,1) share KV head 0 and (2,3) share KV head 1
    np.testing.assert_allclose(sigma[0], (qm[0] + qm[1]) / 2 * km[0], rtol=1e-6)
    np.testing.assert_allclose(sigma[1], (qm[2] + qm[3]) / 2 * km[1], rtol=1e-6)
    # swapping query heads inside a group leaves sigma bit-identical up to fp32 commutativity
    qs = q[[1, 0, 2, 3]].copy()
    _, _, sigma2, _ = orc.score_prefill(cfg, qs, k)
    assert np.array_equal(sigma2, sigma)
    # zeroing group 1's queries zeroes sigma of KV head 1 only
    qz = q.copy()
    qz[2:] = 0
    _, _, sigma3, _ = orc.score_prefill(cfg, qz, k)
    assert np.all(sigma3[1] == 0) and np.array_equal(sigma3[0], sigma[0])
    # n_g = 1: sigma = q_mean * k_mean
    c1 = orc.Cfg(H_q=2, H_kv=2, d=32, pairing=0, n_hi_pairs=4)
    qm1, km1, s1, _ = orc.score_prefill(c1, q[:2], k)
    assert np.array_equal(s1, qm1 * km1)


def test_mean_covers_every_prefill_token(orc):
    """Tokens of every chunk, the ragged tail and the sink positions all count (mean over P)."""
    cfg = orc.Cfg(H_q=1, H_kv=1, d=8, pairing=0, n_hi_pairs=1, g_V=8)
    P = 130
    q = np.zeros((1, P, 8), np.float16)
    k = np.zeros((1, P, 8), np.float16)
    q[0, :, :] = 1.0
    k[0, :, 0] = 1.0            # pair 0: norm 1 on every token
    k[0, 129, 2] = 200.0        # pair 1: one large key in the ragged last chunk
    k[0, 0, 4] = 100.0          # pair 2: one large key at a sink position
    _, km, _, mask = orc.score_prefill(cfg, q.view(np.uint16), k.view(np.uint16))
    np.testing.assert_allclose(km[0], [1.0, 200.0 / P, 100.0 / P, 0.0], rtol=1e-6)
    assert int(mask[0, 0]) == 0b10
