"""CPU oracle for the PN-Mix key-cache data path (ctypes wrapper over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code with the HIP
library in ``decode_attention_pnmix_amd`` and never imports it.

The arithmetic lives in ``pnmix_oracle.c`` (scalar C, IEEE fp32 without contraction, float64
for attention); this module only marshals numpy arrays.  ``joint_causal_score`` is the one
computation written here: the brute-force causal joint score that Eq. 6 approximates
(Korean summary page, "어떻게 동작하나": the separable product of expected query and key pair
norms stands in for the average over causal position pairs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "pnmix_oracle.c")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
            "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class OrcCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "H_q", "H_kv", "d", "pairing", "n_hi_pairs", "G", "b_H", "b_L", "b_V", "g_V", "N_s",
        "N")]


@dataclass(frozen=True)
class Cfg:
    H_q: int
    H_kv: int
    d: int
    pairing: int  # 0 adjacent (2i, 2i+1); 1 split-half (i, i + d/2)
    n_hi_pairs: int
    G: int = 128
    b_H: int = 3
    b_L: int = 1
    b_V: int = 2
    g_V: int = 32
    N_s: int = 32
    N: int = 128

    @property
    def n_g(self) -> int:
        return self.H_q // self.H_kv

    @property
    def n_sal(self) -> int:
        return 2 * self.n_hi_pairs

    def c(self) -> OrcCfg:
        return OrcCfg(self.H_q, self.H_kv, self.d, self.pairing, self.n_hi_pairs, self.G,
                      self.b_H, self.b_L, self.b_V, self.g_V, self.N_s, self.N)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        cp = ctypes.POINTER(OrcCfg)
        sigs = {
            "orc_check_cfg": (ctypes.c_int, [cp]),
            "orc_h2f": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_f2h": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_h2f_array": (None, [P, P, i64]),
            "orc_f2h_array": (None, [P, P, i64]),
            "orc_pair_norm": (ctypes.c_float, [ctypes.c_uint16, ctypes.c_uint16]),
            "orc_pair_norm_array": (None, [P, P, P, i64]),
            "orc_hi_pairs": (i32, [ctypes.c_double, i32]),
            "orc_pair_channels": (None, [cp, i32, P, P]),
            "orc_mask_words": (i32, [cp]),
            "orc_k_page_bytes": (i64, [cp]),
            "orc_v_page_bytes": (i64, [cp]),
            "orc_score_prefill": (ctypes.c_int, [cp, i32, P, P, P, P, P, P]),
            "orc_quantize_k_page": (ctypes.c_int, [cp, P, i64, P, P]),
            "orc_quantize_v_page": (ctypes.c_int, [cp, P, i64, P]),
            "orc_unpack_k_page": (ctypes.c_int, [cp, P, P, P, P, P]),
            "orc_unpack_v_page": (ctypes.c_int, [cp, P, P, P, P]),
            "orc_dequant_k_page": (ctypes.c_int, [cp, P, P, P]),
            "orc_dequant_v_page": (ctypes.c_int, [cp, P, P]),
            "orc_decode_attn_f64": (ctypes.c_int, [cp, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                                   P, ctypes.c_double, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


# ---------------------------------------------------------------------------------------------
# scalar helpers
# ---------------------------------------------------------------------------------------------

def check_cfg(cfg: Cfg) -> bool:
    return lib().orc_check_cfg(ctypes.byref(cfg.c())) == 0


def f2h(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f2h_array(_p(x), _p(out), x.size)
    return out


def h2f(x: np.ndarray) -> np.ndarray:
    x = _u16(x)
    out = np.empty(x.shape, np.float32)
    lib().orc_h2f_array(_p(x), _p(out), x.size)
    return out


def pair_norm(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    x, y = _u16(x), _u16(y)
    assert x.shape == y.shape
    out = np.empty(x.shape, np.float32)
    lib().orc_pair_norm_array(_p(x), _p(y), _p(out), x.size)
    return out


def hi_pairs(r: float, d: int) -> int:
    return int(lib().orc_hi_pairs(float(r), int(d)))


def pair_channels(cfg: Cfg, i: int) -> tuple[int, int]:
    a, b = ctypes.c_int32(), ctypes.c_int32()
    lib().orc_pair_channels(ctypes.byref(cfg.c()), i, ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value


def mask_words(cfg: Cfg) -> int:
    return int(lib().orc_mask_words(ctypes.byref(cfg.c())))


def k_page_bytes(cfg: Cfg) -> int:
    return int(lib().orc_k_page_bytes(ctypes.byref(cfg.c())))


def v_page_bytes(cfg: Cfg) -> int:
    return int(lib().orc_v_page_bytes(ctypes.byref(cfg.c())))


# ---------------------------------------------------------------------------------------------
# the path, one unit at a time
# ---------------------------------------------------------------------------------------------

def score_prefill(cfg: Cfg, q: np.ndarray, k: np.ndarray):
    """One sequence: q [H_q][P][d], k [H_kv][P][d] (fp16 bits).

    Returns (q_mean [H_q][d/2], k_mean [H_kv][d/2], sigma [H_kv][d/2], mask [H_kv][words])."""
    q, k = _u16(q), _u16(k)
    P = q.shape[1]
    assert q.shape == (cfg.H_q, P, cfg.d) and k.shape == (cfg.H_kv, P, cfg.d)
    np_ = cfg.d // 2
    qm = np.empty((cfg.H_q, np_), np.float32)
    km = np.empty((cfg.H_kv, np_), np.float32)
    sg = np.empty((cfg.H_kv, np_), np.float32)
    mk = np.empty((cfg.H_kv, mask_words(cfg)), np.uint32)
    rc = lib().orc_score_prefill(ctypes.byref(cfg.c()), P, _p(q), _p(k), _p(qm), _p(km),
                                 _p(sg), _p(mk))
    if rc:
        raise ValueError("orc_score_prefill rejected its arguments")
    return qm, km, sg, mk


def quantize_k_page(cfg: Cfg, src: np.ndarray, mask_row: np.ndarray) -> np.ndarray:
    src = _u16(src)
    assert src.shape == (cfg.N, cfg.d)
    mask_row = np.ascontiguousarray(mask_row, dtype=np.uint32)
    out = np.empty(k_page_bytes(cfg), np.uint8)
    rc = lib().orc_quantize_k_page(ctypes.byref(cfg.c()), _p(src), cfg.d, _p(mask_row),
                                   _p(out))
    if rc:
        raise ValueError("orc_quantize_k_page rejected its arguments")
    return out


def quantize_v_page(cfg: Cfg, src: np.ndarray) -> np.ndarray:
    src = _u16(src)
    assert src.shape == (cfg.N, cfg.d)
    out = np.empty(v_page_bytes(cfg), np.uint8)
    rc = lib().orc_quantize_v_page(ctypes.byref(cfg.c()), _p(src), cfg.d, _p(out))
    if rc:
        raise ValueError("orc_quantize_v_page rejected its arguments")
    return out


def unpack_k_page(cfg: Cfg, page: np.ndarray, mask_row: np.ndarray):
    page = np.ascontiguousarray(page, dtype=np.uint8)
    mask_row = np.ascontiguousarray(mask_row, dtype=np.uint32)
    codes = np.empty((cfg.N, cfg.d), np.uint8)
    S = np.empty((cfg.N // cfg.G, cfg.d), np.uint16)
    Z = np.empty_like(S)
    rc = lib().orc_unpack_k_page(ctypes.byref(cfg.c()), _p(page), _p(mask_row), _p(codes), _p(S),
                                 _p(Z))
    assert rc == 0
    return codes, S, Z


def unpack_v_page(cfg: Cfg, page: np.ndarray):
    """codes [N][d], S and Z [N][d/g_V] of a quantized value page (b_V < 16)."""
    assert cfg.b_V != 16, "a b_V = 16 page holds fp16 values, not codes"
    page = np.ascontiguousarray(page, dtype=np.uint8)
    codes = np.empty((cfg.N, cfg.d), np.uint8)
    S = np.empty((cfg.N, cfg.d // cfg.g_V), np.uint16)
    Z = np.empty_like(S)
    rc = lib().orc_unpack_v_page(ctypes.byref(cfg.c()), _p(page), _p(codes), _p(S), _p(Z))
    assert rc == 0
    return codes, S, Z


def dequant_k_page(cfg: Cfg, page: np.ndarray, mask_row: np.ndarray) -> np.ndarray:
    page = np.ascontiguousarray(page, dtype=np.uint8)
    mask_row = np.ascontiguousarray(mask_row, dtype=np.uint32)
    out = np.empty((cfg.N, cfg.d), np.float64)
    assert lib().orc_dequant_k_page(ctypes.byref(cfg.c()), _p(page), _p(mask_row), _p(out)) == 0
    return out


def dequant_v_page(cfg: Cfg, page: np.ndarray) -> np.ndarray:
    page = np.ascontiguousarray(page, dtype=np.uint8)
    out = np.empty((cfg.N, cfg.d), np.float64)
    assert lib().orc_dequant_v_page(ctypes.byref(cfg.c()), _p(page), _p(out)) == 0
    return out


def decode_attn_f64(cfg: Cfg, q, k_sink, v_sink, k_pages, v_pages, k_res, v_res, mask,
                    sink_len: int, n_pages: int, res_len: int, sm_scale: float) -> np.ndarray:
    """One sequence.  q [H_q][d]; sinks [H_kv][N_s][d]; pages [H_kv][max_pages][bytes];
    residual [H_kv][N][d]; mask [H_kv][words].  Returns float64 [H_q][d]."""
    q = _u16(q)
    k_sink, v_sink, k_res, v_res = (_u16(a) for a in (k_sink, v_sink, k_res, v_res))
    k_pages = np.ascontiguousarray(k_pages, dtype=np.uint8)
    v_pages = np.ascontiguousarray(v_pages, dtype=np.uint8)
    mask = np.ascontiguousarray(mask, dtype=np.uint32)
    max_pages = k_pages.shape[1]
    assert q.shape == (cfg.H_q, cfg.d)
    assert k_sink.shape == (cfg.H_kv, cfg.N_s, cfg.d) and v_sink.shape == k_sink.shape
    assert k_res.shape == (cfg.H_kv, cfg.N, cfg.d) and v_res.shape == k_res.shape
    assert k_pages.shape == (cfg.H_kv, max_pages, k_page_bytes(cfg))
    assert v_pages.shape == (cfg.H_kv, max_pages, v_page_bytes(cfg))
    out = np.empty((cfg.H_q, cfg.d), np.float64)
    rc = lib().orc_decode_attn_f64(ctypes.byref(cfg.c()), sink_len, n_pages, res_len, max_pages,
                                   _p(q), _p(k_sink), _p(v_sink), _p(k_pages), _p(v_pages),
                                   _p(k_res), _p(v_res), _p(mask), float(sm_scale), _p(out))
    if rc:
        raise ValueError("orc_decode_attn_f64 rejected its arguments")
    return out


def parallel_map(fn, items, threads: int | None = None):
    """Run independent oracle units on a thread pool.  ctypes drops the GIL for the duration
    of each C call, so units run concurrently; results do not depend on the thread count."""
    threads = threads or (os.cpu_count() or 1)
    if threads <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


# ---------------------------------------------------------------------------------------------
# brute-force causal joint score (pin for Eq. 6; tiny inputs only)
# ---------------------------------------------------------------------------------------------

def joint_causal_score(cfg: Cfg, q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Mean over causal position pairs (s <= t) of ||q_{h',t,i}|| * ||k_{h,s,i}||, averaged over
    the query heads h' that share KV head h.  Pure Python loops over (t, s), float64; this is
    the quantity the separable Eq. 6 score approximates (Korean summary page, "어떻게 동작하나").
    Returns [H_kv][d/2]."""
    q = h2f(_u16(q)).astype(np.float64)
    k = h2f(_u16(k)).astype(np.float64)
    P = q.shape[1]
    np_ = cfg.d // 2
    out = np.zeros((cfg.H_kv, np_))
    for h in range(cfg.H_kv):
        for i in range(np_):
            c0, c1 = pair_channels(cfg, i)
            kn = [float(np.hypot(k[h, s, c0], k[h, s, c1])) for s in range(P)]
            tot = 0.0
            for hq in range(h * cfg.n_g, (h + 1) * cfg.n_g):
                acc, cnt = 0.0, 0
                for t in range(P):
                    qn = float(np.hypot(q[hq, t, c0], q[hq, t, c1]))
                    for s in range(t + 1):
                        acc += qn * kn[s]
                        cnt += 1
                tot += acc / cnt
            out[h, i] = tot / cfg.n_g
    return out
