"""ctypes binding of libpnmix.so (include/pnmix.h).  Argument marshalling only.

Every function here takes torch tensors for device memory and torch's current HIP stream, and
passes raw pointers to the C ABI; all arithmetic of the path runs in the library's gfx950
kernels.  There is no fallback: a missing or unloadable library raises immediately.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpnmix.so")

PNMIX_OK, PNMIX_E_INVALID, PNMIX_E_UNSUPPORTED, PNMIX_E_WORKSPACE, PNMIX_E_HIP = range(5)
PAIRS_ADJACENT, PAIRS_SPLIT_HALF = 0, 1


class PnmixError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pnmix status {status}: {msg}")
        self.status = status


class pnmix_cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "H_q", "H_kv", "d", "pairing", "n_hi_pairs", "G", "b_H", "b_L", "b_V", "g_V", "N_s",
        "N")]

    def __repr__(self):
        return "pnmix_cfg(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


def make_cfg(H_q, H_kv, d, pairing, n_hi_pairs, G=128, b_H=3, b_L=1, b_V=2, g_V=32, N_s=32,
             N=128) -> pnmix_cfg:
    return pnmix_cfg(H_q, H_kv, d, pairing, n_hi_pairs, G, b_H, b_L, b_V, g_V, N_s, N)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run decode_attention_pnmix_amd/build.py "
                          "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cp = ctypes.POINTER(pnmix_cfg)
    st = ctypes.c_int
    sigs = {
        "pnmix_check_cfg": (st, [cp]),
        "pnmix_hi_pairs": (i32, [ctypes.c_double, i32]),
        "pnmix_mask_words": (sz, [cp]),
        "pnmix_k_page_bytes": (sz, [cp]),
        "pnmix_v_page_bytes": (sz, [cp]),
        "pnmix_score_workspace_bytes": (sz, [cp, i32, i32]),
        "pnmix_decode_splits": (i32, [cp, i32, i32]),
        "pnmix_decode_plan": (st, [cp, i32, i32, P]),
        "pnmix_decode_workspace_bytes": (sz, [cp, i32, i32]),
        "pnmix_last_error": (ctypes.c_char_p, []),
        "pnmix_score_prefill": (st, [cp, i32, i32, P, P, P, P, P, sz, P]),
        "pnmix_quantize_k_page": (st, [cp, i32, P, P, P]),
        "pnmix_quantize_v_page": (st, [cp, i32, P, P]),
        "pnmix_quantize_kv_pages": (st, [cp, i32, P, P, P, P]),
        "pnmix_prefill_fused_workspace_bytes": (sz, [cp, i32, i32]),
        "pnmix_prefill_fused": (st, [cp, i32, i32, P, P, P, P, P, P, P, i32, P, sz, P]),
        "pnmix_decode_attn": (st, [cp, i32, i32, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P,
                                   sz, P]),
        "pnmix_decode_attn_paged": (st, [cp, i32, i32, P, P, P, P, P, ctypes.c_int64, P, P, P,
                                         P, P, ctypes.c_float, P, P, sz, P]),
        "pnmix_append_decode_attn": (st, [cp, i32, i32] + [P] * 12 + [ctypes.c_float, P, P, sz,
                                                                     P]),
        "pnmix_append_kv": (st, [cp, i32, P, P, P, P, P, P, P, P]),
        "pnmix_commit_page": (st, [cp, i32, i32, P, P]),
        "pnmix_dequant_k_pages": (st, [cp, i32, P, P, P, P]),
        "pnmix_dequant_v_pages": (st, [cp, i32, P, P, P]),
        "pnmix_noalloc_scratch_bytes": (sz, []),
        "pnmix_decode_attn_noalloc": (st, [cp, i32, i32, P, P, P, P, P, P, P, P, P,
                                           ctypes.c_float, P, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


EXPORTED = ("pnmix_check_cfg", "pnmix_hi_pairs", "pnmix_mask_words", "pnmix_k_page_bytes",
            "pnmix_v_page_bytes", "pnmix_score_workspace_bytes", "pnmix_decode_splits",
            "pnmix_decode_plan",
            "pnmix_decode_workspace_bytes", "pnmix_last_error", "pnmix_score_prefill",
            "pnmix_quantize_k_page", "pnmix_quantize_v_page", "pnmix_decode_attn",
            "pnmix_append_kv", "pnmix_commit_page", "pnmix_decode_attn_paged",
            "pnmix_append_decode_attn", "pnmix_dequant_k_pages", "pnmix_dequant_v_pages",
            "pnmix_noalloc_scratch_bytes", "pnmix_decode_attn_noalloc",
            "pnmix_quantize_kv_pages", "pnmix_prefill_fused_workspace_bytes",
            "pnmix_prefill_fused")


def _check(status: int):
    if status != PNMIX_OK:
        raise PnmixError(status, pnmix_last_error())


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("pnmix: tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("pnmix: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _expect(t: torch.Tensor, shape, dtypes, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"pnmix: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"pnmix: {name} has dtype {t.dtype}, expected {dtypes}")


_F16 = (torch.float16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_U32 = (torch.int32, torch.uint32)


# ---- host queries ------------------------------------------------------------------------------

def pnmix_check_cfg(cfg: pnmix_cfg) -> None:
    _check(lib().pnmix_check_cfg(ctypes.byref(cfg)))


def pnmix_hi_pairs(r: float, d: int) -> int:
    return int(lib().pnmix_hi_pairs(float(r), int(d)))


def pnmix_mask_words(cfg) -> int:
    return int(lib().pnmix_mask_words(ctypes.byref(cfg)))


def pnmix_k_page_bytes(cfg) -> int:
    return int(lib().pnmix_k_page_bytes(ctypes.byref(cfg)))


def pnmix_v_page_bytes(cfg) -> int:
    return int(lib().pnmix_v_page_bytes(ctypes.byref(cfg)))


def pnmix_score_workspace_bytes(cfg, B: int, P: int) -> int:
    return int(lib().pnmix_score_workspace_bytes(ctypes.byref(cfg), B, P))


def pnmix_decode_splits(cfg, B: int, max_pages: int) -> int:
    return int(lib().pnmix_decode_splits(ctypes.byref(cfg), B, max_pages))


def pnmix_decode_plan(cfg, B: int, max_pages: int) -> dict:
    """The decode split plan: partials per (sequence, KV head), page waves, fp16-row waves (0:
    their pieces ride on the page waves), waves per workgroup."""
    out = (ctypes.c_int32 * 4)()
    _check(lib().pnmix_decode_plan(ctypes.byref(cfg), B, max_pages, out))
    return {"splits": out[0], "page_splits": out[1], "fp16_splits": out[2], "waves_per_group": out[3]}


def pnmix_decode_workspace_bytes(cfg, B: int, max_pages: int) -> int:
    return int(lib().pnmix_decode_workspace_bytes(ctypes.byref(cfg), B, max_pages))


def pnmix_last_error() -> str:
    return lib().pnmix_last_error().decode()


# ---- the path ----------------------------------------------------------------------------------

def pnmix_score_prefill(cfg, q: torch.Tensor, k: torch.Tensor, sigma: torch.Tensor | None = None,
                        mask: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                        want_sigma: bool = True, stream=None):
    """q [B][H_q][P][d] fp16, k [B][H_kv][P][d] fp16 -> (sigma [B][H_kv][d/2] f32, mask
    [B][H_kv][words] int32 holding the uint32 bit pattern)."""
    B, _, P, _ = q.shape
    _expect(q, (B, cfg.H_q, P, cfg.d), _F16, "q")
    _expect(k, (B, cfg.H_kv, P, cfg.d), _F16, "k")
    dev = q.device
    if mask is None:
        mask = torch.empty(B, cfg.H_kv, pnmix_mask_words(cfg), dtype=torch.int32, device=dev)
    if sigma is None and want_sigma:
        sigma = torch.empty(B, cfg.H_kv, cfg.d // 2, dtype=torch.float32, device=dev)
    need = pnmix_score_workspace_bytes(cfg, B, P)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib().pnmix_score_prefill(ctypes.byref(cfg), B, P, _ptr(q), _ptr(k), _ptr(sigma),
                                     _ptr(mask), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))
    return sigma, mask


def pnmix_prefill_fused_workspace_bytes(cfg, B: int, P: int) -> int:
    return int(lib().pnmix_prefill_fused_workspace_bytes(ctypes.byref(cfg), B, P))


def pnmix_prefill_fused(cfg, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        k_pages: torch.Tensor, v_pages: torch.Tensor,
                        sigma: torch.Tensor | None = None, mask: torch.Tensor | None = None,
                        ws: torch.Tensor | None = None, want_sigma: bool = True, stream=None):
    """Score the prompt and quantize its full pages into slots 0.. of k_pages / v_pages
    [B][max_pages][H_kv][bytes], reading the keys once.  q [B][H_q][P][d], k, v [B][H_kv][P][d]
    fp16 -> (sigma [B][H_kv][d/2] f32, mask [B][H_kv][words])."""
    B, _, P, _ = q.shape
    _expect(q, (B, cfg.H_q, P, cfg.d), _F16, "q")
    _expect(k, (B, cfg.H_kv, P, cfg.d), _F16, "k")
    _expect(v, (B, cfg.H_kv, P, cfg.d), _F16, "v")
    max_pages = k_pages.shape[1]
    _expect(k_pages, (B, max_pages, cfg.H_kv, pnmix_k_page_bytes(cfg)), _U8, "k_pages")
    _expect(v_pages, (B, max_pages, cfg.H_kv, pnmix_v_page_bytes(cfg)), _U8, "v_pages")
    dev = q.device
    if mask is None:
        mask = torch.empty(B, cfg.H_kv, pnmix_mask_words(cfg), dtype=torch.int32, device=dev)
    if sigma is None and want_sigma:
        sigma = torch.empty(B, cfg.H_kv, cfg.d // 2, dtype=torch.float32, device=dev)
    need = pnmix_prefill_fused_workspace_bytes(cfg, B, P)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib().pnmix_prefill_fused(ctypes.byref(cfg), B, P, _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(sigma), _ptr(mask), _ptr(k_pages), _ptr(v_pages),
                                     max_pages, _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))
    return sigma, mask


def page_jobs(src_ptrs, src_row_stride, dst_ptrs, mask_rows, device) -> torch.Tensor:
    """Device array of pnmix_page records {src, src_row_stride, dst, mask_row} (4 x int64)."""
    n = len(dst_ptrs)
    t = torch.empty(n, 4, dtype=torch.int64)
    t[:, 0] = torch.as_tensor(src_ptrs, dtype=torch.int64)
    t[:, 1] = torch.as_tensor(src_row_stride, dtype=torch.int64).expand(n)
    t[:, 2] = torch.as_tensor(dst_ptrs, dtype=torch.int64)
    t[:, 3] = torch.as_tensor(mask_rows, dtype=torch.int64).expand(n)
    return t.to(device)


def pnmix_quantize_k_page(cfg, jobs: torch.Tensor, mask: torch.Tensor, stream=None) -> None:
    _check(lib().pnmix_quantize_k_page(ctypes.byref(cfg), jobs.shape[0], _ptr(jobs), _ptr(mask),
                                       _stream(stream)))


def pnmix_quantize_v_page(cfg, jobs: torch.Tensor, stream=None) -> None:
    _check(lib().pnmix_quantize_v_page(ctypes.byref(cfg), jobs.shape[0], _ptr(jobs),
                                       _stream(stream)))


def pnmix_quantize_kv_pages(cfg, kjobs: torch.Tensor, vjobs: torch.Tensor, mask: torch.Tensor,
                            stream=None) -> None:
    """Key and value page jobs (same count) in one launch."""
    if kjobs.shape != vjobs.shape:
        raise ValueError("pnmix: key and value job arrays differ in shape")
    _check(lib().pnmix_quantize_kv_pages(ctypes.byref(cfg), kjobs.shape[0], _ptr(kjobs),
                                         _ptr(vjobs), _ptr(mask), _stream(stream)))


def pnmix_decode_attn(cfg, q, k_sink, v_sink, k_pages, v_pages, k_res, v_res, lens, mask,
                      sm_scale: float, out: torch.Tensor | None = None,
                      ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [B][H_q][d] fp16; sinks [B][H_kv][N_s][d]; pages [B][max_pages][H_kv][bytes] u8;
    residual [B][H_kv][N][d]; lens [B][4] int32 (sink_len, n_pages, res_len, 0);
    mask [B][H_kv][words] -> out [B][H_q][d] f32.  ws, when given, is a device byte buffer of
    at least pnmix_decode_workspace_bytes(...) bytes that holds the split-K partials."""
    B = q.shape[0]
    max_pages = k_pages.shape[1]
    _expect(q, (B, cfg.H_q, cfg.d), _F16, "q")
    _expect(k_sink, (B, cfg.H_kv, cfg.N_s, cfg.d), _F16, "k_sink")
    _expect(v_sink, (B, cfg.H_kv, cfg.N_s, cfg.d), _F16, "v_sink")
    _expect(k_pages, (B, max_pages, cfg.H_kv, pnmix_k_page_bytes(cfg)), _U8, "k_pages")
    _expect(v_pages, (B, max_pages, cfg.H_kv, pnmix_v_page_bytes(cfg)), _U8, "v_pages")
    _expect(k_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "k_res")
    _expect(v_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "v_res")
    _expect(lens, (B, 4), _U32, "lens")
    _expect(mask, (B, cfg.H_kv, pnmix_mask_words(cfg)), _U32, "mask")
    if out is None:
        out = torch.empty(B, cfg.H_q, cfg.d, dtype=torch.float32, device=q.device)
    need = pnmix_decode_workspace_bytes(cfg, B, max_pages)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().pnmix_decode_attn(ctypes.byref(cfg), B, max_pages, _ptr(q), _ptr(k_sink),
                                   _ptr(v_sink), _ptr(k_pages), _ptr(v_pages), _ptr(k_res),
                                   _ptr(v_res), _ptr(lens), _ptr(mask), float(sm_scale),
                                   _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))
    return out


def pnmix_noalloc_scratch_bytes() -> int:
    return int(lib().pnmix_noalloc_scratch_bytes())


def pnmix_decode_attn_noalloc(cfg, q, k_sink, v_sink, k_pages, v_pages, k_res, v_res, lens, mask,
                              sm_scale: float, out: torch.Tensor, stream=None) -> torch.Tensor:
    """pnmix_decode_attn whose split-K partials live in the library's own device array (the call
    allocates nothing; `out` must be given).  Calls that overlap on one GPU race."""
    B = q.shape[0]
    max_pages = k_pages.shape[1]
    _expect(q, (B, cfg.H_q, cfg.d), _F16, "q")
    _expect(k_sink, (B, cfg.H_kv, cfg.N_s, cfg.d), _F16, "k_sink")
    _expect(v_sink, (B, cfg.H_kv, cfg.N_s, cfg.d), _F16, "v_sink")
    _expect(k_pages, (B, max_pages, cfg.H_kv, pnmix_k_page_bytes(cfg)), _U8, "k_pages")
    _expect(v_pages, (B, max_pages, cfg.H_kv, pnmix_v_page_bytes(cfg)), _U8, "v_pages")
    _expect(k_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "k_res")
    _expect(v_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "v_res")
    _expect(lens, (B, 4), _U32, "lens")
    _expect(mask, (B, cfg.H_kv, pnmix_mask_words(cfg)), _U32, "mask")
    _expect(out, (B, cfg.H_q, cfg.d), (torch.float32,), "out")
    _check(lib().pnmix_decode_attn_noalloc(ctypes.byref(cfg), B, max_pages, _ptr(q), _ptr(k_sink),
                                           _ptr(v_sink), _ptr(k_pages), _ptr(v_pages),
                                           _ptr(k_res), _ptr(v_res), _ptr(lens), _ptr(mask),
                                           float(sm_scale), _ptr(out), _stream(stream)))
    return out


def pnmix_append_decode_attn(cfg, q, k_new, v_new, k_sink, v_sink, k_pages, v_pages, k_res,
                             v_res, lens, lens_out, mask, sm_scale: float,
                             out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                             stream=None) -> torch.Tensor:
    """pnmix_append_kv then pnmix_decode_attn in one call: k_new, v_new [B][H_kv][d] fp16 enter
    the sinks or residual rows, lens [B][4] (before) is read, lens_out [B][4] (after) written."""
    B = q.shape[0]
    max_pages = k_pages.shape[1]
    _expect(q, (B, cfg.H_q, cfg.d), _F16, "q")
    _expect(k_new, (B, cfg.H_kv, cfg.d), _F16, "k_new")
    _expect(v_new, (B, cfg.H_kv, cfg.d), _F16, "v_new")
    _expect(k_sink, (B, cfg.H_kv, cfg.N_s, cfg.d), _F16, "k_sink")
    _expect(v_sink, (B, cfg.H_kv, cfg.N_s, cfg.d), _F16, "v_sink")
    _expect(k_pages, (B, max_pages, cfg.H_kv, pnmix_k_page_bytes(cfg)), _U8, "k_pages")
    _expect(v_pages, (B, max_pages, cfg.H_kv, pnmix_v_page_bytes(cfg)), _U8, "v_pages")
    _expect(k_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "k_res")
    _expect(v_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "v_res")
    _expect(lens, (B, 4), _U32, "lens")
    _expect(lens_out, (B, 4), _U32, "lens_out")
    _expect(mask, (B, cfg.H_kv, pnmix_mask_words(cfg)), _U32, "mask")
    if out is None:
        out = torch.empty(B, cfg.H_q, cfg.d, dtype=torch.float32, device=q.device)
    need = pnmix_decode_workspace_bytes(cfg, B, max_pages)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().pnmix_append_decode_attn(ctypes.byref(cfg), B, max_pages, _ptr(q), _ptr(k_new),
                                          _ptr(v_new), _ptr(k_sink), _ptr(v_sink), _ptr(k_pages),
                                          _ptr(v_pages), _ptr(k_res), _ptr(v_res), _ptr(lens),
                                          _ptr(lens_out), _ptr(mask), float(sm_scale), _ptr(out),
                                          _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream)))
    return out


def pnmix_decode_attn_paged(cfg, q, k_sink, v_sink, k_pool, v_pool, block_table, k_res, v_res,
                            lens, mask, sm_scale: float, out: torch.Tensor | None = None,
                            ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """pnmix_decode_attn over pages held in pools through a block table: k_pool
    [n_blocks][H_kv][k page bytes] u8, v_pool [n_blocks][H_kv][v page bytes] u8, block_table
    [B][max_blocks] int32 (page p of sequence b is block block_table[b][p])."""
    B = q.shape[0]
    max_blocks = block_table.shape[1]
    n_blocks = k_pool.shape[0]
    _expect(q, (B, cfg.H_q, cfg.d), _F16, "q")
    _expect(k_sink, (B, cfg.H_kv, cfg.N_s, cfg.d), _F16, "k_sink")
    _expect(v_sink, (B, cfg.H_kv, cfg.N_s, cfg.d), _F16, "v_sink")
    _expect(k_pool, (n_blocks, cfg.H_kv, pnmix_k_page_bytes(cfg)), _U8, "k_pool")
    _expect(v_pool, (n_blocks, cfg.H_kv, pnmix_v_page_bytes(cfg)), _U8, "v_pool")
    _expect(block_table, (B, max_blocks), _U32, "block_table")
    _expect(k_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "k_res")
    _expect(v_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "v_res")
    _expect(lens, (B, 4), _U32, "lens")
    _expect(mask, (B, cfg.H_kv, pnmix_mask_words(cfg)), _U32, "mask")
    if out is None:
        out = torch.empty(B, cfg.H_q, cfg.d, dtype=torch.float32, device=q.device)
    need = pnmix_decode_workspace_bytes(cfg, B, max_blocks)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().pnmix_decode_attn_paged(ctypes.byref(cfg), B, max_blocks, _ptr(q), _ptr(k_sink),
                                         _ptr(v_sink), _ptr(k_pool), _ptr(v_pool), n_blocks,
                                         _ptr(block_table), _ptr(k_res), _ptr(v_res), _ptr(lens),
                                         _ptr(mask), float(sm_scale), _ptr(out), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)))
    return out


def pnmix_append_kv(cfg, k_new, v_new, k_sink, v_sink, k_res, v_res, lens, stream=None) -> None:
    """k_new, v_new [B][H_kv][d] fp16 -> sink or residual row of each sequence; lens advance on
    the device."""
    B = k_new.shape[0]
    _expect(k_new, (B, cfg.H_kv, cfg.d), _F16, "k_new")
    _expect(v_new, (B, cfg.H_kv, cfg.d), _F16, "v_new")
    _expect(k_res, (B, cfg.H_kv, cfg.N, cfg.d), _F16, "k_res")
    _expect(lens, (B, 4), _U32, "lens")
    _check(lib().pnmix_append_kv(ctypes.byref(cfg), B, _ptr(k_new), _ptr(v_new), _ptr(k_sink),
                                 _ptr(v_sink), _ptr(k_res), _ptr(v_res), _ptr(lens),
                                 _stream(stream)))


def pnmix_dequant_k_pages(cfg, pages: torch.Tensor, mask: torch.Tensor,
                          out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """pages [n][k page bytes] u8, mask [n][words] (the row each page was packed with) ->
    out [n][N][d] f32, x = S code + Z (analysis; decode never forms it)."""
    n = pages.shape[0]
    _expect(pages, (n, pnmix_k_page_bytes(cfg)), _U8, "pages")
    _expect(mask, (n, pnmix_mask_words(cfg)), _U32, "mask")
    if out is None:
        out = torch.empty(n, cfg.N, cfg.d, dtype=torch.float32, device=pages.device)
    _expect(out, (n, cfg.N, cfg.d), (torch.float32,), "out")
    _check(lib().pnmix_dequant_k_pages(ctypes.byref(cfg), n, _ptr(pages), _ptr(mask), _ptr(out),
                                       _stream(stream)))
    return out


def pnmix_dequant_v_pages(cfg, pages: torch.Tensor, out: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """pages [n][v page bytes] u8 -> out [n][N][d] f32 (analysis)."""
    n = pages.shape[0]
    _expect(pages, (n, pnmix_v_page_bytes(cfg)), _U8, "pages")
    if out is None:
        out = torch.empty(n, cfg.N, cfg.d, dtype=torch.float32, device=pages.device)
    _expect(out, (n, cfg.N, cfg.d), (torch.float32,), "out")
    _check(lib().pnmix_dequant_v_pages(ctypes.byref(cfg), n, _ptr(pages), _ptr(out),
                                       _stream(stream)))
    return out


def pnmix_commit_page(cfg, max_pages: int, lens, stream=None) -> None:
    _check(lib().pnmix_commit_page(ctypes.byref(cfg), lens.shape[0], max_pages, _ptr(lens),
                                   _stream(stream)))
