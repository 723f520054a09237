"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: sigma, the pair mask, packed K and V pages (codes and fp16 metadata).
Within max-abs 2e-3 of the float64 oracle: decode attention outputs.
Every workload runs at its full per-layer shape in the launch configuration the benchmark
times; large ones are compared on sampled sequences.  Edge cases: ragged lengths, empty
sequences, full residual buffers, constant / signed-zero / extreme / subnormal groups.
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


# ------------------------------------------------------------------------------- score (Eq. 6)

def _score_case(w, layer, B, P_):
    lc, oc = cfgs(w)
    say(f"[score] {w.name} layer={layer} B={B} P={P_}")
    qp, k, _, _ = layer_inputs(w, layer, B, P_, P_)
    sigma, mask = P.pnmix_score_prefill(lc, qp, k)
    torch.cuda.synchronize()
    qh, kh = u16(qp), u16(k)
    sig_g = sigma.cpu().numpy()
    mask_g = mask.cpu().numpy().view(np.uint32)

    def one(b):
        _, _, s, m = oracle.score_prefill(oc, qh[b], kh[b])
        return s, m

    res = oracle.parallel_map(one, range(B))
    for b, (s, m) in enumerate(res):
        assert np.array_equal(sig_g[b].view(np.uint32), s.view(np.uint32)), f"sigma b={b}"
        assert np.array_equal(mask_g[b], m), f"mask b={b}"
        assert all(sum(bin(int(x)).count("1") for x in m[h]) == w.n_hi_pairs
                   for h in range(w.H_kv))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_score_parity(name):
    w = synth.WORKLOADS[name]
    _score_case(w, 0, w.B, w.P)


def test_score_parity_long_prefill():
    w = synth.WORKLOADS["llama3.1-8b-32L-b110-8k"]
    _score_case(w, 1, 1, w.prefill_score_P)


def test_score_ragged_chunks_and_tiny_P():
    w = synth.WORKLOADS["qwen3-8b-1L-32k"]
    for P_ in (1, 63, 64, 65, 200):
        _score_case(w, 2, 3, P_)


def test_pair_norm_bits_through_score():
    """P = 1 and keys (1, 0) in every pair: sigma = ||q pair|| exactly; random finite fp16 bits
    exercise the fp32 square root and the pair-norm arithmetic bit for bit."""
    d, H = 128, 16
    lc = P.make_cfg(H, H, d, 1, 32)
    oc = oracle.Cfg(H, H, d, 1, 32)
    g = torch.Generator().manual_seed(1)
    B = 512
    bits = torch.randint(0, 1 << 16, (B, H, 1, d), generator=g, dtype=torch.int32)
    bits = torch.where((bits & 0x7C00) == 0x7C00, bits & 0x83FF, bits)  # finite only
    q = bits.to(torch.int16).cuda()
    k = torch.zeros(B, H, 1, d, dtype=torch.float16)
    k[..., :d // 2] = 1.0
    k = k.cuda()
    sigma, _ = P.pnmix_score_prefill(lc, q.view(torch.float16), k)
    torch.cuda.synchronize()
    qh = q.cpu().numpy().view(np.uint16)
    ref = oracle.pair_norm(qh[..., 0, :d // 2], qh[..., 0, d // 2:])
    assert np.array_equal(sigma.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# -------------------------------------------------------------------------- page quantization

def _quant_compare(w, lc, oc, src_gpu, mask_rows_gpu, sample, label):
    """Quantize every page of src [n][N][d] on the GPU; compare `sample` pages with the oracle."""
    n = src_gpu.shape[0]
    kpb, vpb = P.pnmix_k_page_bytes(lc), P.pnmix_v_page_bytes(lc)
    kd = torch.zeros(n, kpb, dtype=torch.uint8, device="cuda")
    vd = torch.zeros(n, vpb, dtype=torch.uint8, device="cuda")
    es = src_gpu.element_size()
    srcs = [src_gpu.data_ptr() + i * w.N * w.d * es for i in range(n)]
    kj = P.page_jobs(srcs, w.d, [kd.data_ptr() + i * kpb for i in range(n)], range(n), "cuda")
    vj = P.page_jobs(srcs, w.d, [vd.data_ptr() + i * vpb for i in range(n)], range(n), "cuda")
    P.pnmix_quantize_k_page(lc, kj, mask_rows_gpu)
    P.pnmix_quantize_v_page(lc, vj)
    # the same jobs as one launch of key and value pages: the same bytes
    kd2, vd2 = torch.zeros_like(kd), torch.zeros_like(vd)
    kj2 = P.page_jobs(srcs, w.d, [kd2.data_ptr() + i * kpb for i in range(n)], range(n), "cuda")
    vj2 = P.page_jobs(srcs, w.d, [vd2.data_ptr() + i * vpb for i in range(n)], range(n), "cuda")
    P.pnmix_quantize_kv_pages(lc, kj2, vj2, mask_rows_gpu)
    torch.cuda.synchronize()
    assert torch.equal(kd, kd2) and torch.equal(vd, vd2), f"{label}: one-launch K+V pages differ"
    sh = u16(src_gpu[sample])
    mh = mask_rows_gpu[sample].cpu().numpy().view(np.uint32)
    kg = kd[sample].cpu().numpy()
    vg = vd[sample].cpu().numpy()

    def one(i):
        return (oracle.quantize_k_page(oc, sh[i], mh[i]), oracle.quantize_v_page(oc, sh[i]))

    res = oracle.parallel_map(one, range(len(sample)))
    for i, (ko, vo) in enumerate(res):
        assert np.array_equal(kg[i], ko), f"{label}: K page {sample[i]} differs"
        assert np.array_equal(vg[i], vo), f"{label}: V page {sample[i]} differs"


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_quant_parity(name):
    w = synth.WORKLOADS[name]
    lc, oc = cfgs(w)
    B = w.B
    T = w.T if w.B * w.H_kv * w.T <= 32 * 8 * 32768 else 8192
    say(f"[quant] {name} B={B} T={T}")
    qp, k, v, _ = layer_inputs(w, 3, B, T)
    _, mask = P.pnmix_score_prefill(lc, qp, k[:, :, :w.P].contiguous())
    n_pages = (T - w.N_s) // w.N
    # pages of keys and of values: [B][H_kv][n_pages][N][d]
    kp = k[:, :, w.N_s:w.N_s + n_pages * w.N].reshape(B, w.H_kv, n_pages, w.N, w.d)
    vp = v[:, :, w.N_s:w.N_s + n_pages * w.N].reshape(B, w.H_kv, n_pages, w.N, w.d)
    rows = mask.reshape(B * w.H_kv, -1)
    mrow = rows.repeat_interleave(n_pages, dim=0).contiguous()
    n = B * w.H_kv * n_pages
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(n, 192), replace=False)]))
    _quant_compare(w, lc, oc, kp.reshape(n, w.N, w.d).contiguous(), mrow, sample, name + "/K")
    # value pages go through the same jobs with the value tokens
    _quant_compare(w, lc, oc, vp.reshape(n, w.N, w.d).contiguous(), mrow, sample, name + "/V")


@pytest.mark.parametrize("G,d,pairing,r,g_V", [(128, 128, 1, 0.5, 32), (64, 128, 1, 0.4, 128),
                                               (32, 64, 0, 0.25, 16), (128, 32, 0, 1.0, 16),
                                               (64, 128, 0, 0.0, 64), (32, 128, 1, 0.5, 32),
                                               (64, 64, 1, 0.5, 64), (32, 32, 1, 0.0, 32)])
def test_quant_adversarial_pages(G, d, pairing, r, g_V):
    """Constant channels and groups, signed zeros, +-65504, subnormals, exact midpoints and
    random finite bit patterns, over every supported token-group and value-group size."""
    w = synth.Workload("adv", 1, 1, 8, 2, d, pairing, 1e4, 64, 512, r, G, g_V=g_V)
    lc, oc = cfgs(w)
    say(f"[quant-adv] G={G} d={d} pairing={pairing} r={r} g_V={g_V}")
    g = torch.Generator().manual_seed(G + d)
    n = 96
    x = torch.randn(n, 128, d, generator=g) * torch.exp(torch.randn(n, 1, d, generator=g) * 2)
    x[0] = 1.25                                   # constant page
    x[1, :, 0] = -0.0
    x[1, 64:, 0] = 0.0                            # {-0, +0} group
    x[2, :, 1] = 65504.0
    x[2, 7, 1] = -65504.0                         # full fp16 range
    x[3] = x[3] * 1e-7                            # subnormal fp16 values
    x[4, :, :] = torch.arange(128).view(128, 1).float() % 8  # exact 3-bit levels
    x[5, :, :] = (torch.arange(128).view(128, 1) % 3).float() * 0.5  # 1-bit midpoints
    x[6, :, : d // 2] = 3.0                       # half of the channels constant
    x[7, ::2] = x[7, 0]                           # tied values
    xh = x.to(torch.float16)
    bits = torch.randint(0, 1 << 16, (8, 128, d), generator=g, dtype=torch.int32)
    bits = torch.where((bits & 0x7C00) == 0x7C00, bits & 0x83FF, bits)
    xh[8:16] = bits.to(torch.int16).view(torch.float16)
    src = xh.cuda().contiguous()
    words = P.pnmix_mask_words(lc)
    nh = w.n_hi_pairs
    masks = torch.zeros(n, words, dtype=torch.int64)
    for i in range(n):
        sel = torch.randperm(d // 2, generator=g)[:nh]
        for p in sel.tolist():
            masks[i, p // 32] |= 1 << (p % 32)
    masks = masks.to(torch.int32).cuda()
    _quant_compare(w, lc, oc, src, masks.contiguous(), np.arange(n), "adversarial")


@pytest.mark.parametrize("pad,offset", [(8, 0), (3, 0), (0, 1), (136, 8), (0, 4)])
def test_quant_strided_sources(pad, offset):
    """Page rows read through a row stride of d + pad elements from a base offset by `offset`
    elements: aligned strides take 16-byte loads, the others 2-byte loads; the packed pages
    must not depend on which."""
    w = synth.WORKLOADS["qwen3-8b-36L-b32-8k"]
    lc, oc = cfgs(w)
    say(f"[quant-stride] pad={pad} offset={offset}")
    g = torch.Generator().manual_seed(pad * 7 + offset)
    n, d = 24, w.d
    stride = d + pad
    flat = (torch.randn(offset + n * w.N * stride, generator=g) *
            torch.exp(torch.randn(offset + n * w.N * stride, generator=g))).to(torch.float16)
    flat_gpu = flat.cuda()
    view = flat[offset:].view(n, w.N, stride)[:, :, :d].contiguous()
    words = P.pnmix_mask_words(lc)
    masks = torch.zeros(n, words, dtype=torch.int64)
    for i in range(n):
        for p in torch.randperm(d // 2, generator=g)[:w.n_hi_pairs].tolist():
            masks[i, p // 32] |= 1 << (p % 32)
    masks = masks.to(torch.int32).cuda()
    kpb, vpb = P.pnmix_k_page_bytes(lc), P.pnmix_v_page_bytes(lc)
    kd = torch.zeros(n, kpb, dtype=torch.uint8, device="cuda")
    vd = torch.zeros(n, vpb, dtype=torch.uint8, device="cuda")
    es = flat_gpu.element_size()
    srcs = [flat_gpu.data_ptr() + (offset + i * w.N * stride) * es for i in range(n)]
    kj = P.page_jobs(srcs, stride, [kd.data_ptr() + i * kpb for i in range(n)], range(n), "cuda")
    vj = P.page_jobs(srcs, stride, [vd.data_ptr() + i * vpb for i in range(n)], range(n), "cuda")
    P.pnmix_quantize_k_page(lc, kj, masks)
    P.pnmix_quantize_v_page(lc, vj)
    torch.cuda.synchronize()
    sh = u16(view)
    mh = masks.cpu().numpy().view(np.uint32)
    kg, vg = kd.cpu().numpy(), vd.cpu().numpy()
    for i in range(n):
        assert np.array_equal(kg[i], oracle.quantize_k_page(oc, sh[i], mh[i])), f"K page {i}"
        assert np.array_equal(vg[i], oracle.quantize_v_page(oc, sh[i])), f"V page {i}"


# ----------------------------------------------------------------------------- decode attention

DECODE_CASES = {
    "tiny": (None, 1),
    "qwen3-8b-1L-32k": (None, 1),
    "qwen3-8b-36L-b32-8k": (None, 4),
    "llama3.1-8b-32L-b110-8k": (None, 4),
    "qwen3-32b-64L-b32-32k": (None, 2),
}


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_decode_parity(name):
    w = synth.WORKLOADS[name]
    lc, oc = cfgs(w)
    _, n_sample = DECODE_CASES[name]
    T = w.T
    say(f"[decode] {name} B={w.B} T={T}")
    qp, k, v, qd = layer_inputs(w, 5, w.B, T)
    cache = fill_cache_bulk(w, lc, qp, k, v, T)
    out = cache.attend(qd)
    torch.cuda.synchronize()
    out_h = out.cpu().numpy()
    mask_g = cache.mask.cpu().numpy().view(np.uint32)
    rng = np.random.default_rng(1)
    picks = sorted(set([0, w.B - 1] + rng.choice(w.B, n_sample, replace=False).tolist()))
    picks = picks[: max(n_sample, 1) + 1]
    for b in picks:
        ref = oracle_decode(w, oc, u16(qp[b]), u16(k[b]), u16(v[b]), u16(qd[b]), T,
                            sm_scale(w.d))
        # the oracle's own mask equals the library's (checked bit-exactly in the score tests)
        err = np.abs(out_h[b] - ref).max()
        say(f"   b={b} max|err|={err:.3e}")
        assert err <= ATOL, (name, b, err)
    del cache, k, v


# value groups of 32 channels take the matrix-core decode kernel, 16-channel groups the generic one
BOTH_KERNELS = pytest.mark.parametrize("g_V", [32, 16], ids=["mfma", "generic"])


def _ragged_case(w, lens_list, max_pages, B=None):
    """Caches built from per-sequence (sink_len, n_pages, res_len), sequences past lens_list
    empty; outputs of the sequences in lens_list against the oracle over the same tokens."""
    lc, oc = cfgs(w)
    d, H_kv = w.d, w.H_kv
    B = B or len(lens_list)
    lens_list = list(lens_list) + [(0, 0, 0)] * (B - len(lens_list))
    Tmax = 32 + max_pages * 128 + 128
    qp, k, v, qd = layer_inputs(w, 0, B, Tmax, 64)
    kpb, vpb = P.pnmix_k_page_bytes(lc), P.pnmix_v_page_bytes(lc)
    _, mask = P.pnmix_score_prefill(lc, qp, k[:, :, :64].contiguous())
    k_sink = torch.zeros(B, H_kv, 32, d, dtype=torch.float16, device="cuda")
    v_sink = torch.zeros_like(k_sink)
    k_res = torch.zeros(B, H_kv, 128, d, dtype=torch.float16, device="cuda")
    v_res = torch.zeros_like(k_res)
    k_pages = torch.zeros(B, max_pages, H_kv, kpb, dtype=torch.uint8, device="cuda")
    v_pages = torch.zeros(B, max_pages, H_kv, vpb, dtype=torch.uint8, device="cuda")
    lens = torch.zeros(B, 4, dtype=torch.int32)
    srcs, kd, vd, rows, vsrcs = [], [], [], [], []
    for b, (s, npg, r) in enumerate(lens_list):
        lens[b, :3] = torch.tensor([s, npg, r])
        k_sink[b, :, :s] = k[b, :, :s]
        v_sink[b, :, :s] = v[b, :, :s]
        for h in range(H_kv):
            for p in range(npg):
                off = ((b * H_kv + h) * Tmax + 32 + p * 128) * d * 2
                srcs.append(k.data_ptr() + off)
                vsrcs.append(v.data_ptr() + off)
                kd.append(k_pages.data_ptr() + ((b * max_pages + p) * H_kv + h) * kpb)
                vd.append(v_pages.data_ptr() + ((b * max_pages + p) * H_kv + h) * vpb)
                rows.append(b * H_kv + h)
        a = 32 + npg * 128
        k_res[b, :, :r] = k[b, :, a:a + r]
        v_res[b, :, :r] = v[b, :, a:a + r]
    if srcs:
        P.pnmix_quantize_k_page(lc, P.page_jobs(srcs, d, kd, rows, "cuda"), mask)
        P.pnmix_quantize_v_page(lc, P.page_jobs(vsrcs, d, vd, rows, "cuda"))
    out = P.pnmix_decode_attn(lc, qd, k_sink, v_sink, k_pages, v_pages, k_res, v_res,
                              lens.cuda(), mask, sm_scale(d))
    torch.cuda.synchronize()
    out_h = out.cpu().numpy()
    mask_h = mask.cpu().numpy().view(np.uint32)
    kh, vh = u16(k), u16(v)
    for b, (s, npg, r) in enumerate(lens_list):
        if s + npg + r == 0:
            assert np.all(out_h[b] == 0)
            continue
        # the oracle places the same token ranges itself
        kp = np.zeros((H_kv, max_pages, kpb), np.uint8)
        vp = np.zeros((H_kv, max_pages, vpb), np.uint8)
        for h in range(H_kv):
            for p in range(npg):
                a = 32 + p * 128
                kp[h, p] = oracle.quantize_k_page(oc, kh[b, h, a:a + 128], mask_h[b, h])
                vp[h, p] = oracle.quantize_v_page(oc, vh[b, h, a:a + 128])
        ks = np.zeros((H_kv, 32, d), np.uint16)
        vs = np.zeros_like(ks)
        ks[:, :s] = kh[b, :, :s]
        vs[:, :s] = vh[b, :, :s]
        a = 32 + npg * 128
        kr = np.zeros((H_kv, 128, d), np.uint16)
        vr = np.zeros_like(kr)
        kr[:, :r] = kh[b, :, a:a + r]
        vr[:, :r] = vh[b, :, a:a + r]
        ref = oracle.decode_attn_f64(oc, u16(qd[b]), ks, vs, kp, vp, kr, vr, mask_h[b], s, npg,
                                     r, sm_scale(d))
        err = np.abs(out_h[b] - ref).max()
        assert err <= ATOL, (lens_list[b], err)


@BOTH_KERNELS
def test_decode_ragged_lengths_and_edges(g_V):
    """Per-sequence lengths in one batch: empty, sinks only, partial sinks, residual only, full
    residual (N rows), pages with and without residual, n_pages = max_pages."""
    w = synth.Workload("ragged", 1, 1, 8, 2, 64, 1, 1e4, 64, 1024, 0.5, 64, g_V=g_V)
    lens_list = [(0, 0, 0), (5, 0, 0), (32, 0, 0), (32, 0, 77), (32, 0, 128), (32, 1, 0),
                 (32, 3, 1), (32, 7, 128), (32, 7, 0), (32, 2, 64)]
    say(f"[decode-ragged] B={len(lens_list)}")
    _ragged_case(w, lens_list, 7)


def test_decode_ragged_fp16_pieces_on_page_waves():
    """A large batch (256 (sequence, KV head) items, d = 128, 4 query heads per KV head: two
    waves per SIMD) with a long capacity, where the plan puts the fp16 rows' 32-token pieces on
    the page waves (no fp16 waves of their own: one round of resident waves, not two): ragged
    lengths (no pages, few pages, one residual row, full residual, full capacity, empty
    sequences) against the oracle."""
    w = synth.Workload("ragged-spread", 1, 1, 8, 2, 128, 1, 1e6, 64, 1024, 0.5, 128)
    lc, _ = cfgs(w)
    B, max_pages = 128, 255
    plan = P.pnmix_decode_plan(lc, B, max_pages)
    say(f"[decode-ragged-spread] B={B} plan={plan}")
    assert plan["fp16_splits"] == 0 and plan["waves_per_group"] == 1
    lens_list = [(0, 0, 0), (5, 0, 0), (32, 0, 0), (32, 0, 77), (32, 0, 128), (32, 1, 0),
                 (32, 3, 1), (32, 255, 128), (32, 255, 0), (32, 2, 64), (32, 7, 5),
                 (32, 254, 100), (32, 8, 31), (32, 100, 17), (17, 0, 0)]
    _ragged_case(w, lens_list, max_pages, B)


def test_decode_split_count_does_not_change_results():
    """The same sequence alone (many splits) and inside a batch of 64 (fewer splits).  B = 1
    takes the small-batch plan (several waves per workgroup, one page split each, their
    partials merged on chip); B = 64 the large-batch plan (one wave per workgroup, a few page
    splits, the fp16 rows folded into the last one); both then go through the merge launch."""
    w = synth.WORKLOADS["qwen3-8b-1L-32k"]
    lc, _ = cfgs(w)
    T = 4096 + 32 + 50
    qp, k, v, qd = layer_inputs(w, 7, 1, T)
    c1 = fill_cache_bulk(w, lc, qp, k, v, T)
    o1 = c1.attend(qd)
    B = 64
    c2 = fill_cache_bulk(w, lc, qp.expand(B, -1, -1, -1).contiguous(),
                         k.expand(B, -1, -1, -1).contiguous(),
                         v.expand(B, -1, -1, -1).contiguous(), T)
    o2 = c2.attend(qd.expand(B, -1, -1).contiguous())
    torch.cuda.synchronize()
    n1 = P.pnmix_decode_splits(lc, 1, c1.max_pages)
    n2 = P.pnmix_decode_splits(lc, B, c2.max_pages)
    assert n1 >= 2 and n2 >= 2
    assert torch.equal(c1.k_pages[0], c2.k_pages[B - 1])
    assert (o2 - o1).abs().max().item() <= 1e-5


# ------------------------------------------------------------------------ online vs bulk fill

ONLINE_CASES = {
    "tiny": (synth.WORKLOADS["tiny"], {65, 159, 160, 161, 288, 289, 512}),
    # d = 128 split-half pairs, 4 query heads per KV head, G = 64, B = 2, P = 141: page flushes
    # at 160, 288 and 416 cached tokens
    "d128-G64": (synth.Workload("online-d128", 1, 2, 16, 4, 128, 1, 1e6, 141, 436, 0.5, 64),
                 {142, 159, 160, 161, 288, 289, 416, 417, 436}),
}


@pytest.mark.parametrize("name", list(ONLINE_CASES))
def test_online_fill_equals_bulk_fill(name):
    """Prefill P tokens, then one decode step at a time (attend, then quantize when the residual
    buffer is full): every packed page equals bulk quantization of the same tokens, and outputs
    match the oracle along the way."""
    w, checks = ONLINE_CASES[name]
    lc, oc = cfgs(w)
    T = w.T
    max_pages = (T - w.N_s) // w.N + 1
    qp, k, v, _ = layer_inputs(w, 0, w.B, T)
    npairs = w.d // 2
    sq = synth.pair_scales(w.H_q, npairs, w.sigma_ln, "cuda", w.name, 0, "q")
    c = P.PNMixLayerCache(lc, w.B, max_pages)
    c.prefill(qp, k[:, :, :w.P].contiguous(), v[:, :, :w.P].contiguous())
    assert c.n_score_calls == 1
    mask0 = c.mask.clone()
    say(f"[online] {name} B={w.B} P={w.P} T={T}")
    for t in range(w.P, T):
        qt = synth.rope_tokens(sq, w.B, torch.tensor([t], device="cuda"), w.d, w.pairing,
                               w.rope_base, "cuda", w.name, 0, "qstep", t)[:, :, 0].contiguous()
        o = c.step(qt, k[:, :, t].contiguous(), v[:, :, t].contiguous())
        if t + 1 in checks:
            torch.cuda.synchronize()
            for b in range(w.B):
                ref = oracle_decode(w, oc, u16(qp[b]), u16(k[b]), u16(v[b]), u16(qt[b]), t + 1,
                                    sm_scale(w.d), online=True)
                assert np.abs(o[b].cpu().numpy() - ref).max() <= ATOL, (t + 1, b)
    assert c.n_score_calls == 1 and torch.equal(c.mask, mask0)  # mask fixed after prefill
    bulk = fill_cache_bulk(w, lc, qp, k, v, T, max_pages=max_pages)
    torch.cuda.synchronize()
    assert (c.sink_len, c.n_pages, c.res_len) == (bulk.sink_len, bulk.n_pages, bulk.res_len)
    assert torch.equal(c.k_pages[:, :c.n_pages], bulk.k_pages[:, :bulk.n_pages])
    assert torch.equal(c.v_pages[:, :c.n_pages], bulk.v_pages[:, :bulk.n_pages])
    assert torch.equal(c.k_sink, bulk.k_sink)
    assert torch.equal(c.k_res[:, :, :c.res_len], bulk.k_res[:, :, :bulk.res_len])


# ------------------------------------------------------------ decode kernel instantiations

# Small shapes that reach every split-kernel variant the supported configurations select:
# head tiles (4-head tiles: 1, 2, and 4 for up to 16 heads, a partly empty second tile for
# 6 heads), key groups per page (G = 128, 64, 32), one or two upper-bit K-steps (r > 0.5 gives
# more than 64 salient channels at d = 128; r = 0 and r = 1 are the all-1-bit and all-3-bit key
# caches), d in {32, 64, 128}, and both launch shapes
# (workgroups of several waves merged on chip for fewer than 128 (sequence, KV head) items,
# one wave per workgroup otherwise).  T = 466 holds sinks, three pages and 50 residual rows.
INST_CASES = [
    # id, H_q, H_kv, d, pairing, r, G, g_V, B
    ("ng8-G64", 16, 2, 128, 1, 0.5, 64, 32, 2),
    ("ng8-G64-B64", 16, 2, 128, 1, 0.5, 64, 32, 64),
    ("ng4-r075", 8, 2, 128, 1, 0.75, 128, 32, 2),
    ("ng8-r075", 16, 2, 128, 1, 0.75, 128, 32, 2),
    ("ng16", 32, 2, 128, 1, 0.5, 128, 32, 2),
    ("ng6-G32", 12, 2, 128, 0, 0.5, 32, 32, 2),
    ("d64-ng8", 16, 2, 64, 0, 0.5, 128, 32, 2),
    ("d32-ng12", 24, 2, 32, 0, 0.25, 64, 16, 2),
    ("ng4-B64", 8, 2, 128, 1, 0.5, 128, 32, 64),
    ("ng4-r0", 8, 2, 128, 1, 0.0, 128, 32, 2),
    ("ng4-r1", 8, 2, 128, 1, 1.0, 128, 32, 2),
    ("tinyshape-r0", 4, 2, 32, 0, 0.0, 128, 32, 1),
]


@pytest.mark.parametrize("case", INST_CASES, ids=[c[0] for c in INST_CASES])
def test_decode_instantiations(case):
    name, H_q, H_kv, d, pairing, r, G, g_V, B = case
    T = 32 + 3 * 128 + 50
    w = synth.Workload(name, 1, B, H_q, H_kv, d, pairing, 1e4, 64, T, r, G, g_V=g_V)
    lc, oc = cfgs(w)
    say(f"[decode-inst] {name} B={B} splits={P.pnmix_decode_splits(lc, B, w.n_pages)}")
    qp, k, v, qd = layer_inputs(w, 3, B, T)
    cache = fill_cache_bulk(w, lc, qp, k, v, T)
    out = cache.attend(qd)
    torch.cuda.synchronize()
    out_h = out.cpu().numpy()
    for b in sorted({0, B // 2, B - 1}):
        ref = oracle_decode(w, oc, u16(qp[b]), u16(k[b]), u16(v[b]), u16(qd[b]), T,
                            sm_scale(d))
        err = np.abs(out_h[b] - ref).max()
        say(f"   b={b} max|err|={err:.3e}")
        assert err <= ATOL, (name, b, err)


# ------------------------------------------------------------------------- paged page pools

PAGED_CASES = [
    # id, workload, B, T, spare table columns, ragged page counts
    ("qwen3-8b-B1", "qwen3-8b-1L-32k", 1, 32 + 20 * 128 + 77, 0, False),
    ("qwen3-32b-B3", "qwen3-32b-64L-b32-32k", 3, 32 + 5 * 128 + 9, 3, True),
    ("qwen3-8b-B8", "qwen3-8b-36L-b32-8k", 8, 32 + 6 * 128 + 128, 2, True),
    ("llama-B40", "llama3.1-8b-32L-b110-8k", 40, 32 + 4 * 128 + 1, 0, True),
    # 128 (sequence, KV head) items and 201 pages: the plan spreads the fp16 pieces over the
    # page waves
    ("qwen3-32b-B16-spread", "qwen3-32b-64L-b32-32k", 16, 32 + 200 * 128 + 50, 1, True),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_paged_decode_equals_contiguous(case):
    """The same pages scattered over a shuffled block pool and read through a block table give
    the same outputs, bit for bit, as the contiguous page arrays (same kernels, same split
    plan).  Pool blocks no table entry names hold random bytes; table entries past a sequence's
    page count hold junk (negative or past the pool), which is never used."""
    name, wname, B, T, spare, ragged = case
    w = synth.WORKLOADS[wname]
    lc, _ = cfgs(w)
    qp, k, v, qd = layer_inputs(w, 4, B, T)
    n_pages = (T - w.N_s) // w.N
    c = fill_cache_bulk(w, lc, qp, k, v, T, max_pages=n_pages + spare)
    if "spread" in name:
        plan = P.pnmix_decode_plan(lc, B, c.max_pages)
        say(f"[paged] {name} plan={plan}")
        assert plan["fp16_splits"] == 0 and plan["waves_per_group"] == 1
    if ragged:  # fewer pages for some sequences (their residual rows stay)
        for b in range(0, B, 2):
            c.lens[b, 1] = (b // 2) % (n_pages + 1)
    out_c = c.attend(qd)
    H, mp = w.H_kv, c.max_pages
    n_blocks = B * mp + 7
    gen = torch.Generator().manual_seed(11)
    perm = torch.randperm(n_blocks, generator=gen)[:B * mp].reshape(B, mp)
    kpb, vpb = P.pnmix_k_page_bytes(lc), P.pnmix_v_page_bytes(lc)
    k_pool = torch.randint(0, 256, (n_blocks, H, kpb), dtype=torch.uint8, generator=gen).cuda()
    v_pool = torch.randint(0, 256, (n_blocks, H, vpb), dtype=torch.uint8, generator=gen).cuda()
    idx = perm[:, :n_pages].reshape(-1).cuda()
    k_pool[idx] = c.k_pages[:, :n_pages].reshape(-1, H, kpb)
    v_pool[idx] = c.v_pages[:, :n_pages].reshape(-1, H, vpb)
    table = perm.to(torch.int32).clone()
    table[:, n_pages:] = torch.where(torch.arange(spare) % 2 == 0, -5, n_blocks + 100)
    out_p = P.pnmix_decode_attn_paged(lc, qd, c.k_sink, c.v_sink, k_pool, v_pool, table.cuda(),
                                      c.k_res, c.v_res, c.lens, c.mask, c.sm_scale)
    torch.cuda.synchronize()
    say(f"[paged] {name} B={B} pages={n_pages} table={mp} blocks={n_blocks}")
    assert torch.equal(out_p, out_c)
    # against the oracle: the first sequence and the last, and a ragged one (fewer pages, the
    # same residual rows), each placed by the oracle from the fp16 tokens
    _, oc = cfgs(w)
    lens_h = c.lens.cpu().numpy()
    mask_h = c.mask.cpu().numpy().view(np.uint32)
    out_h = out_p.cpu().numpy()
    kh, vh = u16(k), u16(v)
    picks = sorted({0, B - 1} | ({2} if ragged and B > 2 else set()))
    res0 = w.N_s + n_pages * w.N
    for b in picks:
        s_, npg, r = (int(x) for x in lens_h[b, :3])
        kp = np.zeros((H, max(npg, 1), kpb), np.uint8)
        vp = np.zeros((H, max(npg, 1), vpb), np.uint8)
        for h in range(H):
            for p in range(npg):
                a = w.N_s + p * w.N
                kp[h, p] = oracle.quantize_k_page(oc, kh[b, h, a:a + w.N], mask_h[b, h])
                vp[h, p] = oracle.quantize_v_page(oc, vh[b, h, a:a + w.N])
        ks = np.zeros((H, w.N_s, w.d), np.uint16)
        vs = np.zeros_like(ks)
        ks[:, :s_], vs[:, :s_] = kh[b, :, :s_], vh[b, :, :s_]
        kr = np.zeros((H, w.N, w.d), np.uint16)
        vr = np.zeros_like(kr)
        kr[:, :r], vr[:, :r] = kh[b, :, res0:res0 + r], vh[b, :, res0:res0 + r]
        ref = oracle.decode_attn_f64(oc, u16(qd[b]), ks, vs, kp, vp, kr, vr, mask_h[b], s_, npg,
                                     r, sm_scale(w.d))
        err = np.abs(out_h[b] - ref).max()
        say(f"   b={b} lens={s_, npg, r} max|err|={err:.3e}")
        assert err <= ATOL, (name, b, err)


@BOTH_KERNELS
def test_decode_without_pages_both_entry_points(g_V):
    """max_pages = 0 (sinks and residual rows only): both decode entry points, against the
    oracle, with ragged sink and residual counts."""
    w = synth.Workload("nopages", 1, 1, 8, 2, 64, 1, 1e4, 64, 1024, 0.5, 64, g_V=g_V)
    lc, oc = cfgs(w)
    lens_list = [(0, 0, 0), (7, 0, 0), (32, 0, 0), (32, 0, 1), (32, 0, 128), (32, 0, 65)]
    B = len(lens_list)
    say(f"[decode-nopages] B={B}")
    qp, k, v, qd = layer_inputs(w, 2, B, 32 + 128, 64)
    _, mask = P.pnmix_score_prefill(lc, qp, k[:, :, :64].contiguous())
    k_sink = torch.zeros(B, 2, 32, 64, dtype=torch.float16, device="cuda")
    v_sink = torch.zeros_like(k_sink)
    k_res = torch.zeros(B, 2, 128, 64, dtype=torch.float16, device="cuda")
    v_res = torch.zeros_like(k_res)
    lens = torch.zeros(B, 4, dtype=torch.int32)
    for b, (s_, _, r) in enumerate(lens_list):
        lens[b, :3] = torch.tensor([s_, 0, r])
        k_sink[b, :, :s_] = k[b, :, :s_]
        v_sink[b, :, :s_] = v[b, :, :s_]
        k_res[b, :, :r] = k[b, :, 32:32 + r]
        v_res[b, :, :r] = v[b, :, 32:32 + r]
    lens = lens.cuda()
    kp0 = torch.zeros(B, 0, 2, P.pnmix_k_page_bytes(lc), dtype=torch.uint8, device="cuda")
    vp0 = torch.zeros(B, 0, 2, P.pnmix_v_page_bytes(lc), dtype=torch.uint8, device="cuda")
    out_c = P.pnmix_decode_attn(lc, qd, k_sink, v_sink, kp0, vp0, k_res, v_res, lens, mask,
                                sm_scale(64))
    kpool = torch.zeros(1, 2, P.pnmix_k_page_bytes(lc), dtype=torch.uint8, device="cuda")
    vpool = torch.zeros(1, 2, P.pnmix_v_page_bytes(lc), dtype=torch.uint8, device="cuda")
    table = torch.zeros(B, 0, dtype=torch.int32, device="cuda")
    out_p = P.pnmix_decode_attn_paged(lc, qd, k_sink, v_sink, kpool, vpool, table, k_res, v_res,
                                      lens, mask, sm_scale(64))
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p)
    out_h = out_c.cpu().numpy()
    mask_h = mask.cpu().numpy().view(np.uint32)
    kh, vh = u16(k), u16(v)
    for b, (s_, _, r) in enumerate(lens_list):
        if s_ + r == 0:
            assert np.all(out_h[b] == 0)
            continue
        ks = np.zeros((2, 32, 64), np.uint16)
        vs = np.zeros_like(ks)
        ks[:, :s_] = kh[b, :, :s_]
        vs[:, :s_] = vh[b, :, :s_]
        kr = np.zeros((2, 128, 64), np.uint16)
        vr = np.zeros_like(kr)
        kr[:, :r] = kh[b, :, 32:32 + r]
        vr[:, :r] = vh[b, :, 32:32 + r]
        kp = np.zeros((2, 0, P.pnmix_k_page_bytes(lc)), np.uint8)
        vp = np.zeros((2, 0, P.pnmix_v_page_bytes(lc)), np.uint8)
        ref = oracle.decode_attn_f64(oc, u16(qd[b]), ks, vs, kp, vp, kr, vr, mask_h[b], s_, 0,
                                     r, sm_scale(64))
        err = np.abs(out_h[b] - ref).max()
        assert err <= ATOL, (lens_list[b], err)


@BOTH_KERNELS
def test_fused_step_equals_append_then_attend(g_V):
    """pnmix_append_decode_attn (the cache's step) against pnmix_append_kv + pnmix_decode_attn,
    bit for bit, from a 5-token prompt: sinks filling, residual rows, a page flush; then a
    sequence whose residual buffer is full takes no new row."""
    w = synth.Workload("fused", 1, 2, 8, 2, 64, 1, 1e4, 5, 5 + 200, 0.5, 64, g_V=g_V)
    lc, _ = cfgs(w)
    T = w.T
    max_pages = (T - w.N_s) // w.N + 1
    qp, k, v, _ = layer_inputs(w, 1, w.B, T)
    sq = synth.pair_scales(w.H_q, w.d // 2, w.sigma_ln, "cuda", w.name, 1, "q")
    c1 = P.PNMixLayerCache(lc, w.B, max_pages)
    c2 = P.PNMixLayerCache(lc, w.B, max_pages)
    for c in (c1, c2):
        c.prefill(qp, k[:, :, :w.P].contiguous(), v[:, :, :w.P].contiguous())
    say(f"[fused] B={w.B} P={w.P} T={T}")
    for t in range(w.P, T):
        qt = synth.rope_tokens(sq, w.B, torch.tensor([t], device="cuda"), w.d, w.pairing,
                               w.rope_base, "cuda", w.name, 1, "qstep", t)[:, :, 0].contiguous()
        kt, vt = k[:, :, t].contiguous(), v[:, :, t].contiguous()
        o1 = c1.step(qt, kt, vt)
        c2.append(kt, vt)
        o2 = c2.attend(qt)
        c2.flush()
        assert torch.equal(o1, o2), t
    torch.cuda.synchronize()
    assert (c1.sink_len, c1.n_pages, c1.res_len) == (c2.sink_len, c2.n_pages, c2.res_len)
    assert c1.n_pages == 1 and c1.sink_len == w.N_s
    for name in ("lens", "k_sink", "v_sink", "k_res", "v_res", "k_pages", "v_pages"):
        assert torch.equal(getattr(c1, name), getattr(c2, name)), name
    # residual buffer full for sequence 1: no row is placed and its lengths stay
    lens_full = c2.lens.clone()
    lens_full[1, 2] = w.N
    k_res0, lens_out = c2.k_res.clone(), torch.full_like(lens_full, -7)
    kt, vt = k[:, :, 3].contiguous(), v[:, :, 3].contiguous()
    qt = synth.rope_tokens(sq, w.B, torch.tensor([T], device="cuda"), w.d, w.pairing,
                           w.rope_base, "cuda", w.name, 1, "qstep", T)[:, :, 0].contiguous()
    ref = P.pnmix_decode_attn(lc, qt, c2.k_sink, c2.v_sink, c2.k_pages, c2.v_pages, c2.k_res,
                              c2.v_res, lens_full, c2.mask, c2.sm_scale)
    torch.cuda.synchronize()
    out = P.pnmix_append_decode_attn(lc, qt, kt, vt, c2.k_sink, c2.v_sink, c2.k_pages,
                                     c2.v_pages, c2.k_res, c2.v_res, lens_full, lens_out,
                                     c2.mask, c2.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out[1], ref[1])
    assert torch.equal(lens_out[1], lens_full[1])
    assert torch.equal(c2.k_res[1], k_res0[1])
    r0 = int(lens_full[0, 2])
    assert int(lens_out[0, 2]) == r0 + 1 and torch.equal(c2.k_res[0, :, r0], kt[0])


def test_decode_many_splits():
    """One long sequence of a 2-KV-head model (640 pages at d = 128): more than 64 partials per
    (sequence, KV head), so each merge lane folds its splits in several rounds of eight loads."""
    T = 32 + 640 * 128 + 17
    w = synth.Workload("many-splits", 1, 1, 8, 2, 128, 1, 1e6, 141, T, 0.5, 128)
    lc, oc = cfgs(w)
    n_splits = P.pnmix_decode_splits(lc, 1, (T - w.N_s) // w.N)
    say(f"[decode-many-splits] T={T} splits={n_splits}")
    assert n_splits > 64
    qp, k, v, qd = layer_inputs(w, 9, 1, T)
    cache = fill_cache_bulk(w, lc, qp, k, v, T)
    out = cache.attend(qd)
    torch.cuda.synchronize()
    ref = oracle_decode(w, oc, u16(qp[0]), u16(k[0]), u16(v[0]), u16(qd[0]), T, sm_scale(w.d))
    err = np.abs(out[0].cpu().numpy() - ref).max()
    say(f"   max|err|={err:.3e}")
    assert err <= ATOL


FUSED_ORACLE_CASES = [
    # workload, sampled sequences: one fused step over T - 1 cached tokens -> T tokens
    ("qwen3-8b-1L-32k", (0,)),
    ("qwen3-32b-64L-b32-32k", (0, 17, 31)),
]


@pytest.mark.parametrize("wname,picks", FUSED_ORACLE_CASES, ids=[c[0] for c in FUSED_ORACLE_CASES])
def test_fused_step_against_the_oracle(wname, picks):
    """pnmix_append_decode_attn (what the benchmark times) at full shape: a cache of T - 1 tokens
    (bulk filled), then one fused step appends token T - 1 and attends over all T; the outputs of
    sampled sequences are within 2e-3 of the float64 oracle over the same T tokens, and the new
    rows and lengths are in place."""
    w = synth.WORKLOADS[wname]
    lc, oc = cfgs(w)
    T = w.T
    say(f"[fused-oracle] {wname} B={w.B} T={T}")
    qp, k, v, qd = layer_inputs(w, 12, w.B, T)
    c = fill_cache_bulk(w, lc, qp, k, v, T - 1, max_pages=(T - w.N_s) // w.N + 1)
    out = c.step(qd, k[:, :, T - 1].contiguous(), v[:, :, T - 1].contiguous())
    torch.cuda.synchronize()
    assert (c.sink_len, c.n_pages, c.res_len) == (w.N_s, w.n_pages, w.res_len)
    assert torch.equal(c.lens[:, :3].cpu(), torch.tensor([[w.N_s, w.n_pages, w.res_len]] * w.B,
                                                          dtype=torch.int32))
    assert torch.equal(c.k_res[:, :, w.res_len - 1], k[:, :, T - 1])
    out_h = out.cpu().numpy()
    for b in picks:
        ref = oracle_decode(w, oc, u16(qp[b]), u16(k[b]), u16(v[b]), u16(qd[b]), T,
                            sm_scale(w.d))
        err = np.abs(out_h[b] - ref).max()
        say(f"   b={b} max|err|={err:.3e}")
        assert err <= ATOL, (wname, b, err)


def test_score_folded_batch_above_65535():
    """Layers folded into the batch: 1,700 sequences x (32 + 8) heads = 68,000 (sequence, head)
    rows of Llama-3.1-8B shape, beyond a grid y dimension; sampled sequences bit-exact."""
    w = synth.WORKLOADS["llama3.1-8b-32L-b110-8k"]
    lc, oc = cfgs(w)
    B, P_ = 1700, 24
    say(f"[score-folded] B={B} P={P_}")
    qp, k, _, _ = layer_inputs(w, 0, B, P_, P_)
    sigma, mask = P.pnmix_score_prefill(lc, qp, k)
    torch.cuda.synchronize()
    for b in (0, 977, B - 1):
        _, _, s, m = oracle.score_prefill(oc, u16(qp[b]), u16(k[b]))
        assert np.array_equal(sigma[b].cpu().numpy().view(np.uint32), s.view(np.uint32)), b
        assert np.array_equal(mask[b].cpu().numpy().view(np.uint32), m), b


# ----------------------------------------------------------------- fused prefill (one key read)

PREFILL_CASES = [
    # id, workload, B, P
    ("qwen3-8b-P141-B32", "qwen3-8b-36L-b32-8k", 32, 141),   # no full page: score only
    ("qwen3-8b-ragged-P", "qwen3-8b-1L-32k", 2, None),        # several P, see below
    ("tiny-d32", "tiny", 3, 32 + 2 * 128 + 40),
    ("llama-G64-P2000", "llama3.1-8b-32L-b110-8k", 2, 2000),
]


def _prefill_check(w, B, P_):
    lc, oc = cfgs(w)
    qp, k, v, _ = layer_inputs(w, 13, B, P_, P_)
    n_full = max(0, (P_ - w.N_s) // w.N)
    mp = max(n_full, 1)
    kp1 = torch.zeros(B, mp, w.H_kv, P.pnmix_k_page_bytes(lc), dtype=torch.uint8, device="cuda")
    vp1 = torch.zeros(B, mp, w.H_kv, P.pnmix_v_page_bytes(lc), dtype=torch.uint8, device="cuda")
    sig_f, mask_f = P.pnmix_prefill_fused(lc, qp, k, v, kp1, vp1)
    # the unfused sequence: score, then both page kinds in one launch
    sig_u, mask_u = P.pnmix_score_prefill(lc, qp, k)
    c = P.PNMixLayerCache(lc, B, mp)
    c.mask.copy_(mask_u)
    if n_full:
        kj, _ = c.page_jobs(k, w.N_s, 0, n_full)
        _, vj = c.page_jobs(v, w.N_s, 0, n_full)
        P.pnmix_quantize_kv_pages(lc, kj, vj, c.mask)
    torch.cuda.synchronize()
    assert torch.equal(sig_f.view(torch.int32), sig_u.view(torch.int32))
    assert torch.equal(mask_f, mask_u)
    assert torch.equal(kp1[:, :n_full], c.k_pages[:, :n_full])
    assert torch.equal(vp1[:, :n_full], c.v_pages[:, :n_full])
    # against the oracle: the mask of sampled sequences and some of their pages
    mh = mask_f.cpu().numpy().view(np.uint32)
    kh, vh = u16(k), u16(v)
    for b in sorted({0, B - 1}):
        _, _, s, m = oracle.score_prefill(oc, u16(qp[b]), kh[b])
        assert np.array_equal(sig_f[b].cpu().numpy().view(np.uint32), s.view(np.uint32)), b
        assert np.array_equal(mh[b], m), b
        for p in sorted({0, n_full - 1, n_full // 2}) if n_full else []:
            for h in (0, w.H_kv - 1):
                a = w.N_s + p * w.N
                assert np.array_equal(kp1[b, p, h].cpu().numpy(),
                                      oracle.quantize_k_page(oc, kh[b, h, a:a + w.N], m[h])), (b, p, h)
                assert np.array_equal(vp1[b, p, h].cpu().numpy(),
                                      oracle.quantize_v_page(oc, vh[b, h, a:a + w.N])), (b, p, h)
    return n_full


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_fused(case):
    name, wname, B, P_ = case
    w = synth.WORKLOADS[wname]
    # prompt lengths around the chunk and page boundaries: pages end mid-chunk or on a chunk
    # boundary, and the chunks after the last page may be empty, partial or full
    lengths = [P_] if P_ else [32 + 128, 32 + 128 + 1, 32 + 2 * 128 + 31, 32 + 2 * 128 + 32,
                               32 + 2 * 128 + 33, 32 + 3 * 128 + 95, 32 + 3 * 128 + 96, 31, 33]
    for L_ in lengths:
        n_full = _prefill_check(w, B, L_)
        say(f"[prefill-fused] {name} B={B} P={L_} pages={n_full}")


@pytest.mark.parametrize("n_s", [0, 16, 64, 96])
def test_prefill_fused_sink_offsets(n_s):
    """Sink counts that put the pages on, or off, the 64-token chunk grid: the page workgroups
    add up exactly the key chunks lying inside their page and the score kernel the others."""
    import dataclasses
    w = dataclasses.replace(synth.WORKLOADS["qwen3-8b-1L-32k"], name=f"sinks{n_s}", N_s=n_s)
    for L_ in (n_s + 3 * 128 + 40, n_s + 2 * 128):
        n_full = _prefill_check(w, 2, L_)
        say(f"[prefill-fused] N_s={n_s} P={L_} pages={n_full}")


def test_prefill_fused_long_prompt():
    """The 16K-token prompt at B = 1 (Llama-3.1-8B shape, G = 64, r = 0.4): 127 pages per KV head."""
    w = synth.WORKLOADS["llama3.1-8b-32L-b110-8k"]
    n_full = _prefill_check(w, 1, w.prefill_score_P)
    say(f"[prefill-fused] llama 16K pages={n_full}")
    assert n_full == (w.prefill_score_P - w.N_s) // w.N
