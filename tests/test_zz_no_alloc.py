"""pnmix_decode_attn_noalloc (the decode entry point that allocates nothing) against
pnmix_decode_attn with a caller workspace, through the C ABI: bit-identical outputs on two calls
in a row, the second on a smaller batch with fewer pages (the library's scratch array keeps the
first call's partials; nothing in it may leak into the second), on both decode kernels."""
import numpy as np
import pytest
import torch

import decode_attention_pnmix_amd as P
import oracle
import synth
from _cases import cfgs, fill_cache_bulk, layer_inputs, oracle_decode, say, sm_scale, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    P.lib()


def _call_both(w, lc, B, T, layer):
    qp, k, v, qd = layer_inputs(w, layer, B, T)
    c = fill_cache_bulk(w, lc, qp, k, v, T)
    ref = c.attend(qd)
    out = torch.full_like(ref, float("nan"))
    P.pnmix_decode_attn_noalloc(lc, qd, c.k_sink, c.v_sink, c.k_pages, c.v_pages, c.k_res,
                                c.v_res, c.lens, c.mask, c.sm_scale, out)
    torch.cuda.synchronize()
    return out, ref, (qp, k, v, qd)


@pytest.mark.parametrize("bH,bL", [(3, 1), (4, 2)], ids=["mfma", "generic"])
def test_noalloc_equals_workspace_call_twice(bH, bL):
    w = synth.Workload("noalloc", 1, 32, 32, 8, 128, 1, 1e6, 141, 32 + 40 * 128 + 77, 0.5, 128,
                       b_H=bH, b_L=bL)
    lc, oc = cfgs(w)
    big_B, big_T = 32, w.T
    say(f"[noalloc] b_H={bH} b_L={bL} first call B={big_B} T={big_T}")
    o1, r1, inp = _call_both(w, lc, big_B, big_T, 0)
    assert torch.equal(o1, r1)
    # ... against the oracle too, on one sequence
    qp, k, v, qd = inp
    ref = oracle_decode(w, oc, u16(qp[5]), u16(k[5]), u16(v[5]), u16(qd[5]), big_T,
                        sm_scale(w.d))
    assert np.abs(o1[5].cpu().numpy() - ref).max() <= 2e-3
    say(f"[noalloc] b_H={bH} b_L={bL} second call B=3 T=300")
    o2, r2, _ = _call_both(w, lc, 3, 300, 1)
    assert torch.equal(o2, r2)
