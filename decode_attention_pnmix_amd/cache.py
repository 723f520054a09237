"""Online cache policy for one attention layer of B sequences (the harness around the ABI).

PN-Mix paper (arXiv 2610.19605) sec. 2 and sec. 5: new keys and values enter an FP16 residual
buffer of N tokens; when it is full it is quantized and appended to the quantized cache; the
first N_s tokens of every sequence (sinks) are never quantized; the pair mask comes from the
prefill score once and is reused for every page.  This class tracks the lengths on the host
(for its own decisions), copies the prompt's fp16 rows into place at prefill, and otherwise only
calls library entry points (score, page quantization, append, commit, decode); it holds no
arithmetic.

Reading taken where the pages are silent: in the step where the residual buffer reaches N
tokens, the step attends first and quantizes afterwards, so attention always sees between 1
and N residual rows.  All sequences of one cache advance together (equal lengths).
"""
from __future__ import annotations

import math

import torch

from . import _lib as L


class PNMixLayerCache:
    def __init__(self, cfg: L.pnmix_cfg, B: int, max_pages: int, device="cuda"):
        L.pnmix_check_cfg(cfg)
        self.cfg, self.B, self.max_pages, self.device = cfg, B, max_pages, device
        H, d = cfg.H_kv, cfg.d
        f16 = torch.float16
        self.k_sink = torch.zeros(B, H, cfg.N_s, d, dtype=f16, device=device)
        self.v_sink = torch.zeros_like(self.k_sink)
        # pages [B][max_pages][H_kv][bytes]: page p of every KV head side by side
        self.k_pages = torch.zeros(B, max_pages, H, L.pnmix_k_page_bytes(cfg), dtype=torch.uint8,
                                   device=device)
        self.v_pages = torch.zeros(B, max_pages, H, L.pnmix_v_page_bytes(cfg), dtype=torch.uint8,
                                   device=device)
        self.k_res = torch.zeros(B, H, cfg.N, d, dtype=f16, device=device)
        self.v_res = torch.zeros_like(self.k_res)
        self.mask = torch.zeros(B, H, L.pnmix_mask_words(cfg), dtype=torch.int32, device=device)
        self.sigma = None
        self.sink_len = self.n_pages = self.res_len = 0
        self.lens = torch.zeros(B, 4, dtype=torch.int32, device=device)
        self._lens_next = torch.zeros_like(self.lens)  # lengths written by a fused step
        self.sm_scale = float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
        self.ws = torch.empty(max(L.pnmix_decode_workspace_bytes(cfg, B, max_pages), 256),
                              dtype=torch.uint8, device=device)
        self.n_score_calls = 0
        self._flush_jobs = {}

    # -- helpers -------------------------------------------------------------------------------
    def _sync_lens(self):
        self.lens[:, 0] = self.sink_len
        self.lens[:, 1] = self.n_pages
        self.lens[:, 2] = self.res_len

    def page_jobs(self, src: torch.Tensor, first_token: int, page_slot: int, n: int = 1):
        """Jobs quantizing tokens [first_token + i N, ...) of src [B][H_kv][T][d] into page
        slots page_slot + i, i < n, for every (sequence, KV head)."""
        cfg, B, H = self.cfg, self.B, self.cfg.H_kv
        es = src.element_size()
        kpb, vpb = self.k_pages.shape[-1], self.v_pages.shape[-1]
        srcs, kd, vd, rows = [], [], [], []
        base = src.data_ptr()
        T, d = src.shape[2], src.shape[3]
        for b in range(B):
            for h in range(H):
                for i in range(n):
                    srcs.append(base + (((b * H + h) * T) + first_token + i * cfg.N) * d * es)
                    slot = (b * self.max_pages + page_slot + i) * H + h
                    kd.append(self.k_pages.data_ptr() + slot * kpb)
                    vd.append(self.v_pages.data_ptr() + slot * vpb)
                    rows.append(b * H + h)
        kj = L.page_jobs(srcs, d, kd, rows, self.device)
        vj = L.page_jobs(srcs, d, vd, rows, self.device)
        return kj, vj

    # -- policy --------------------------------------------------------------------------------
    def prefill(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, fused: bool = False):
        """Score the prompt once (Eq. 6), keep sinks, quantize full pages, keep the rest fp16.
        fused: score and quantize the prompt's pages in one pass over the keys
        (pnmix_prefill_fused, same bytes; (b_H, b_L, b_V) = (3, 1, 2) only)."""
        cfg = self.cfg
        P = k.shape[2]
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("prefill keys and values must be contiguous [B][H_kv][P][d]")
        s = min(P, cfg.N_s)
        n_full = (P - s) // cfg.N
        if n_full > self.max_pages:
            raise ValueError("prompt exceeds the cache capacity")
        if fused:
            self.sigma, mask = L.pnmix_prefill_fused(cfg, q, k, v, self.k_pages, self.v_pages)
            self.mask.copy_(mask)
        else:
            self.sigma, mask = L.pnmix_score_prefill(cfg, q, k)
            self.mask.copy_(mask)
        self.n_score_calls += 1
        self.k_sink[:, :, :s] = k[:, :, :s]
        self.v_sink[:, :, :s] = v[:, :, :s]
        if n_full and not fused:
            kj, _ = self.page_jobs(k, s, 0, n_full)
            _, vj = self.page_jobs(v, s, 0, n_full)
            L.pnmix_quantize_kv_pages(cfg, kj, vj, self.mask)
            torch.cuda.current_stream().synchronize()  # jobs reference k, v
        rest = P - s - n_full * cfg.N
        a = s + n_full * cfg.N
        self.k_res[:, :, :rest] = k[:, :, a:]
        self.v_res[:, :, :rest] = v[:, :, a:]
        self.sink_len, self.n_pages, self.res_len = s, n_full, rest
        self._sync_lens()

    def load_context(self, q_prompt: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        """A cache holding a whole context at once: the mask is scored on the first P tokens
        (q_prompt [B][H_q][P][d] against k[:, :, :P]), then k, v [B][H_kv][T][d] are placed as
        sinks, full pages (bulk quantization) and an fp16 residual of the remaining rows.  The
        result equals filling the cache one decode step at a time after a P-token prefill
        whenever every page boundary was crossed by a flush."""
        cfg = self.cfg
        P, T = q_prompt.shape[2], k.shape[2]
        if not (k.is_contiguous() and v.is_contiguous()):
            raise ValueError("keys and values must be contiguous [B][H_kv][T][d]")
        if P > T:
            raise ValueError("the prompt is longer than the context")
        self.sigma, mask = L.pnmix_score_prefill(cfg, q_prompt, k[:, :, :P].contiguous())
        self.mask.copy_(mask)
        self.n_score_calls += 1
        s = min(T, cfg.N_s)
        n_full = (T - s) // cfg.N
        if n_full > self.max_pages:
            raise ValueError("context exceeds the cache capacity")
        self.k_sink.zero_()
        self.v_sink.zero_()
        self.k_sink[:, :, :s] = k[:, :, :s]
        self.v_sink[:, :, :s] = v[:, :, :s]
        if n_full:
            kj, _ = self.page_jobs(k, s, 0, n_full)
            _, vj = self.page_jobs(v, s, 0, n_full)
            L.pnmix_quantize_kv_pages(cfg, kj, vj, self.mask)
            torch.cuda.current_stream().synchronize()  # jobs reference k, v
        a = s + n_full * cfg.N
        rest = T - a
        self.k_res.zero_()
        self.v_res.zero_()
        self.k_res[:, :, :rest] = k[:, :, a:]
        self.v_res[:, :, :rest] = v[:, :, a:]
        self.sink_len, self.n_pages, self.res_len = s, n_full, rest
        self._sync_lens()

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor):
        """k_new, v_new [B][H_kv][d]: the decode step's key and value, placed by the library
        (sink row while the sinks are filling, else the next residual row)."""
        cfg = self.cfg
        if self.res_len >= cfg.N:
            raise RuntimeError("residual buffer full: flush() after attending")
        L.pnmix_append_kv(cfg, k_new, v_new, self.k_sink, self.v_sink, self.k_res, self.v_res,
                          self.lens)
        if self.sink_len < cfg.N_s and self.n_pages == 0 and self.res_len == 0:
            self.sink_len += 1
        else:
            self.res_len += 1

    def attend(self, q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        return L.pnmix_decode_attn(self.cfg, q, self.k_sink, self.v_sink, self.k_pages,
                                   self.v_pages, self.k_res, self.v_res, self.lens, self.mask,
                                   self.sm_scale, out=out, ws=self.ws)

    def flush_jobs(self, slot: int):
        """Page jobs that quantize the residual buffers into page `slot` (built once)."""
        if slot not in self._flush_jobs:
            kj, _ = self.page_jobs(self.k_res, 0, slot)
            _, vj = self.page_jobs(self.v_res, 0, slot)
            self._flush_jobs[slot] = (kj, vj)
        return self._flush_jobs[slot]

    def flush(self):
        """Quantize the residual buffer into the next page once it holds N tokens."""
        cfg = self.cfg
        if self.res_len < cfg.N:
            return False
        if self.n_pages >= self.max_pages:
            raise RuntimeError("cache capacity exhausted")
        kj, vj = self.flush_jobs(self.n_pages)
        L.pnmix_quantize_kv_pages(cfg, kj, vj, self.mask)
        L.pnmix_commit_page(cfg, self.max_pages, self.lens)
        self.n_pages += 1
        self.res_len = 0
        return True

    def step(self, q, k_new, v_new, out=None):
        """One decode step: append and attend in one call (pnmix_append_decode_attn, the same
        outputs as append then attend), then quantize if the residual buffer is full."""
        cfg = self.cfg
        if self.res_len >= cfg.N:
            raise RuntimeError("residual buffer full: flush() after attending")
        o = L.pnmix_append_decode_attn(cfg, q, k_new, v_new, self.k_sink, self.v_sink,
                                       self.k_pages, self.v_pages, self.k_res, self.v_res,
                                       self.lens, self._lens_next, self.mask, self.sm_scale,
                                       out=out, ws=self.ws)
        self.lens, self._lens_next = self._lens_next, self.lens
        if self.sink_len < cfg.N_s and self.n_pages == 0 and self.res_len == 0:
            self.sink_len += 1
        else:
            self.res_len += 1
        self.flush()
        return o
