"""The C ABI on a machine without a GPU: the library loads, exports every declared symbol,
validates arguments on the host before any HIP call, and reports a missing device as
PNMIX_E_HIP (no CPU fallback)."""
import ctypes
import os
import re

import pytest

import decode_attention_pnmix_amd as P
from decode_attention_pnmix_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pnmix.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pnmix_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = P.lib()
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


def _cfg(**kw):
    base = dict(H_q=32, H_kv=8, d=128, pairing=1, n_hi_pairs=32, G=128, b_H=3, b_L=1, b_V=2,
                g_V=32, N_s=32, N=128)
    base.update(kw)
    return L.pnmix_cfg(*[base[n] for n, _ in L.pnmix_cfg._fields_])


@pytest.mark.parametrize("kw,status", [
    ({}, L.PNMIX_OK),
    ({"H_q": 30}, L.PNMIX_E_INVALID),
    ({"H_q": 8 * 17}, L.PNMIX_E_UNSUPPORTED),
    ({"d": 96}, L.PNMIX_E_UNSUPPORTED),
    ({"d": 33}, L.PNMIX_E_INVALID),
    ({"pairing": 2}, L.PNMIX_E_INVALID),
    ({"n_hi_pairs": 65}, L.PNMIX_E_INVALID),
    ({"n_hi_pairs": -1}, L.PNMIX_E_INVALID),
    ({"G": 48}, L.PNMIX_E_INVALID),
    ({"G": 16}, L.PNMIX_E_UNSUPPORTED),
    ({"b_H": 4, "b_L": 2}, L.PNMIX_OK),
    ({"b_H": 1, "b_L": 1}, L.PNMIX_OK),
    ({"b_H": 2, "b_L": 3}, L.PNMIX_E_INVALID),
    ({"b_H": 5, "b_L": 1}, L.PNMIX_E_UNSUPPORTED),
    ({"b_L": 0}, L.PNMIX_E_INVALID),
    ({"b_V": 4}, L.PNMIX_OK),
    ({"b_V": 16}, L.PNMIX_OK),
    ({"b_V": 3}, L.PNMIX_E_UNSUPPORTED),
    ({"g_V": 24}, L.PNMIX_E_INVALID),
    ({"g_V": 16}, L.PNMIX_E_UNSUPPORTED),
    ({"d": 64, "g_V": 16}, L.PNMIX_OK),
    ({"N": 64}, L.PNMIX_E_UNSUPPORTED),
    ({"N_s": -1}, L.PNMIX_E_INVALID),
    ({"d": 32, "g_V": 32, "n_hi_pairs": 8, "pairing": 0, "H_q": 4, "H_kv": 2}, L.PNMIX_OK),
])
def test_check_cfg(kw, status):
    st = P.lib().pnmix_check_cfg(ctypes.byref(_cfg(**kw)))
    assert st == status, P.pnmix_last_error()
    if status != L.PNMIX_OK:
        assert P.pnmix_last_error()


def test_sizes_match_the_oracle(orc):
    for d, r, G, g_V, bH, bL, bV in ((128, 0.5, 128, 32, 3, 1, 2), (128, 0.4, 64, 32, 3, 1, 2),
                                     (32, 0.5, 128, 32, 3, 1, 2), (64, 0.25, 32, 16, 3, 1, 2),
                                     (128, 0.3, 64, 32, 4, 2, 16), (64, 0.6, 128, 16, 4, 3, 4),
                                     (128, 0.5, 32, 64, 2, 2, 1), (32, 0.9, 64, 32, 4, 1, 16)):
        n_hi = P.pnmix_hi_pairs(r, d)
        assert n_hi == orc.hi_pairs(r, d)
        c = _cfg(d=d, n_hi_pairs=n_hi, G=G, g_V=g_V, b_H=bH, b_L=bL, b_V=bV)
        oc = orc.Cfg(32, 8, d, 1, n_hi, G=G, g_V=g_V, b_H=bH, b_L=bL, b_V=bV)
        assert P.pnmix_k_page_bytes(c) == orc.k_page_bytes(oc)
        assert P.pnmix_v_page_bytes(c) == orc.v_page_bytes(oc)
        assert P.pnmix_mask_words(c) == orc.mask_words(oc)
    assert P.pnmix_hi_pairs(0.4, 128) == 25
    assert P.pnmix_hi_pairs(0.0, 128) == 0 and P.pnmix_hi_pairs(1.0, 128) == 64


def test_decode_plan_queries():
    c = _cfg()
    for B, mp in ((1, 255), (32, 63), (110, 63), (1, 0), (4, 3)):
        s = P.pnmix_decode_splits(c, B, mp)
        # partials per (sequence, KV head): page splits (at most one per page) plus the fp16
        # splits (one in all for large batches, at most one per 64-token chunk of the sink and
        # residual rows for small ones), several splits per workgroup for small batches
        n16_max = 1 if B * c.H_kv >= 128 else (c.N_s + c.N + 63) // 64
        assert 1 <= s <= min(mp + n16_max, 136)
        assert P.pnmix_decode_workspace_bytes(c, B, mp) >= B * 8 * s * 4 * (128 + 2) * 4
        plan = P.pnmix_decode_plan(c, B, mp)
        nw = plan["waves_per_group"]
        assert plan["splits"] == s == -(-(plan["page_splits"] + plan["fp16_splits"]) // nw)
        assert plan["page_splits"] <= mp
        # no fp16 waves: only with pages, one wave per workgroup and a large batch
        if plan["fp16_splits"] == 0:
            assert mp > 0 and nw == 1 and B * c.H_kv >= 128
    assert P.pnmix_decode_splits(_cfg(G=48), 1, 10) == 0
    for args in ((_cfg(G=48), 1, 10), (c, 0, 10), (c, 1, -1)):
        with pytest.raises(P.PnmixError):
            P.pnmix_decode_plan(*args)
    # the generic kernel (other bit widths): one split per 128-token chunk at most
    for kw in ({"b_V": 16}, {"b_H": 4, "b_L": 2}, {"d": 64, "g_V": 16}):
        for B, mp in ((1, 255), (32, 63), (1, 0)):
            s = P.pnmix_decode_splits(_cfg(**kw), B, mp)
            assert 1 <= s <= min(mp + 2, 136)


def test_noalloc_rejects_oversized_batches_before_any_launch():
    """pnmix_decode_attn_noalloc's partials live in the library's fixed device array: a batch
    that needs more is refused with PNMIX_E_WORKSPACE and a message, before any HIP call."""
    lib = P.lib()
    cap = P.pnmix_noalloc_scratch_bytes()
    assert cap == 32 << 20
    c = _cfg()
    big = 4096
    assert P.pnmix_decode_workspace_bytes(c, big, 255) > cap
    args = [FAKE] * 9
    st = lib.pnmix_decode_attn_noalloc(ctypes.byref(c), big, 255, *args, ctypes.c_float(0.088),
                                       FAKE, None)
    assert st == L.PNMIX_E_WORKSPACE
    assert "scratch" in P.pnmix_last_error()
    assert lib.pnmix_decode_attn_noalloc(ctypes.byref(c), 4, 10, None, *args[1:],
                                         ctypes.c_float(0.088), FAKE, None) == L.PNMIX_E_INVALID


def test_prefill_fused_validation_before_launch():
    lib = P.lib()
    c = _cfg()
    B, P_ = 2, 32 + 3 * 128 + 5
    ws = P.pnmix_prefill_fused_workspace_bytes(c, B, P_)
    assert ws >= P.pnmix_score_workspace_bytes(c, B, P_) + B * 8 * 3 * (128 * 128 // 2)

    def call(cfg=c, max_pages=3, ws_bytes=ws, k_pages=FAKE):
        return lib.pnmix_prefill_fused(ctypes.byref(cfg), B, P_, FAKE, FAKE, FAKE, None, FAKE,
                                       k_pages, FAKE, max_pages, FAKE, ws_bytes, None)

    assert call(cfg=_cfg(b_V=4)) == L.PNMIX_E_UNSUPPORTED
    assert call(max_pages=2) == L.PNMIX_E_INVALID  # the prompt fills 3 pages
    assert call(ws_bytes=ws - 1) == L.PNMIX_E_WORKSPACE
    assert call(k_pages=None) == L.PNMIX_E_INVALID
    assert P.pnmix_last_error()


def test_score_accepts_a_folded_batch_above_65535():
    """Layers fold into the batch: Llama-3.1-8B's 32 layers x B = 110 x (32 + 8) heads is 140,800
    (sequence, head) rows, above the 65,535 limit of a grid's y dimension.  Validation passes;
    without a device the launch then reports PNMIX_E_HIP."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present (this checks host validation only)")
    c = _cfg(n_hi_pairs=25, G=64)
    B = 32 * 110
    ws = P.pnmix_score_workspace_bytes(c, B, 141)
    assert ws > 0
    st = P.lib().pnmix_score_prefill(ctypes.byref(c), B, 141, FAKE, FAKE, None, FAKE, FAKE, ws,
                                     None)
    assert st == L.PNMIX_E_HIP, P.pnmix_last_error()


FAKE = ctypes.c_void_p(0x10000)


def test_validation_before_launch():
    lib = P.lib()
    c = _cfg()
    ws = P.pnmix_score_workspace_bytes(c, 2, 141)
    assert ws > 0 and ws % 256 == 0
    # null inputs
    assert lib.pnmix_score_prefill(ctypes.byref(c), 2, 141, None, FAKE, None, FAKE, FAKE, ws,
                                   None) == L.PNMIX_E_INVALID
    # workspace too small
    assert lib.pnmix_score_prefill(ctypes.byref(c), 2, 141, FAKE, FAKE, None, FAKE, FAKE, ws - 1,
                                   None) == L.PNMIX_E_WORKSPACE
    assert lib.pnmix_score_prefill(ctypes.byref(c), 0, 141, FAKE, FAKE, None, FAKE, FAKE, ws,
                                   None) == L.PNMIX_E_INVALID
    assert lib.pnmix_quantize_k_page(ctypes.byref(c), 4, None, FAKE, None) == L.PNMIX_E_INVALID
    assert lib.pnmix_quantize_k_page(ctypes.byref(c), -1, FAKE, FAKE, None) == L.PNMIX_E_INVALID
    assert lib.pnmix_quantize_v_page(ctypes.byref(c), 0, None, None) == L.PNMIX_OK
    dws = P.pnmix_decode_workspace_bytes(c, 4, 10)
    args = [FAKE] * 9
    assert lib.pnmix_decode_attn(ctypes.byref(c), 4, 10, *args, ctypes.c_float(0.088), FAKE,
                                 FAKE, dws - 1, None) == L.PNMIX_E_WORKSPACE
    assert lib.pnmix_decode_attn(ctypes.byref(c), 4, 10, *args, ctypes.c_float(float("nan")),
                                 FAKE, FAKE, dws, None) == L.PNMIX_E_INVALID
    assert lib.pnmix_decode_attn(ctypes.byref(c), 4, 10, None, *args[1:],
                                 ctypes.c_float(0.088), FAKE, FAKE, dws,
                                 None) == L.PNMIX_E_INVALID
    assert lib.pnmix_decode_attn(ctypes.byref(_cfg(b_V=3)), 4, 10, *args, ctypes.c_float(0.1),
                                 FAKE, FAKE, dws, None) == L.PNMIX_E_UNSUPPORTED
    # one sequence's contiguous pages must span less than 2 GiB (one buffer resource)
    big = 2**31 // (8 * P.pnmix_v_page_bytes(c)) + 1
    assert lib.pnmix_decode_attn(ctypes.byref(c), 1, big, *args, ctypes.c_float(0.088), FAKE,
                                 FAKE, P.pnmix_decode_workspace_bytes(c, 1, big),
                                 None) == L.PNMIX_E_UNSUPPORTED
    assert "2 GiB" in P.pnmix_last_error()


def test_paged_validation_before_launch():
    lib = P.lib()
    c = _cfg()
    dws = P.pnmix_decode_workspace_bytes(c, 4, 10)

    def call(max_blocks=10, n_blocks=40, table=FAKE, k_pool=FAKE, ws_bytes=dws, cfg=c, B=4):
        return lib.pnmix_decode_attn_paged(ctypes.byref(cfg), B, max_blocks, FAKE, FAKE, FAKE,
                                           k_pool, FAKE, n_blocks, table, FAKE, FAKE, FAKE, FAKE,
                                           ctypes.c_float(0.088), FAKE, FAKE, ws_bytes, None)

    assert call(table=None) == L.PNMIX_E_INVALID
    assert call(k_pool=None) == L.PNMIX_E_INVALID
    assert call(n_blocks=0) == L.PNMIX_E_INVALID
    assert call(max_blocks=-1) == L.PNMIX_E_INVALID
    assert call(B=0) == L.PNMIX_E_INVALID
    assert call(ws_bytes=dws - 1) == L.PNMIX_E_WORKSPACE
    assert call(cfg=_cfg(b_V=3)) == L.PNMIX_E_UNSUPPORTED
    assert P.pnmix_last_error()


def test_fused_step_validation_before_launch():
    lib = P.lib()
    c = _cfg()
    dws = P.pnmix_decode_workspace_bytes(c, 4, 10)

    def call(k_new=FAKE, lens=FAKE, lens_out=ctypes.c_void_p(0x20000)):
        return lib.pnmix_append_decode_attn(ctypes.byref(c), 4, 10, FAKE, k_new, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, FAKE, lens, lens_out, FAKE,
                                            ctypes.c_float(0.088), FAKE, FAKE, dws, None)

    assert call(k_new=None) == L.PNMIX_E_INVALID
    assert call(lens_out=None) == L.PNMIX_E_INVALID
    assert call(lens_out=FAKE) == L.PNMIX_E_INVALID  # lens_out is lens
    assert call(lens_out=ctypes.c_void_p(0x10000 + 16)) == L.PNMIX_E_INVALID  # overlapping
    assert "overlap" in P.pnmix_last_error()


def test_no_device_is_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = P.lib()
    c = _cfg()
    ws = P.pnmix_score_workspace_bytes(c, 1, 141)
    st = lib.pnmix_score_prefill(ctypes.byref(c), 1, 141, FAKE, FAKE, None, FAKE, FAKE, ws, None)
    assert st == L.PNMIX_E_HIP
    assert "HIP error" in P.pnmix_last_error()
