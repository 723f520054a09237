"""MI355X-native PN-Mix key-cache data path.

The compute lives in libpnmix.so (hand-written gfx950 HIP kernels behind the C ABI of
include/pnmix.h); this package is its Python binding (argument marshalling over torch device
memory and streams) plus the online cache policy around it.
"""
from ._lib import (PAIRS_ADJACENT, PAIRS_SPLIT_HALF, PnmixError, lib, make_cfg, page_jobs,
                   pnmix_append_decode_attn, pnmix_append_kv, pnmix_cfg, pnmix_commit_page, pnmix_check_cfg, pnmix_decode_attn,
                   pnmix_decode_attn_paged, pnmix_decode_plan, pnmix_decode_splits,
                   pnmix_decode_attn_noalloc, pnmix_decode_workspace_bytes, pnmix_dequant_k_pages,
                   pnmix_dequant_v_pages, pnmix_noalloc_scratch_bytes,
                   pnmix_hi_pairs, pnmix_k_page_bytes,
                   pnmix_last_error, pnmix_mask_words, pnmix_quantize_k_page,
                   pnmix_prefill_fused, pnmix_prefill_fused_workspace_bytes,
                   pnmix_quantize_kv_pages, pnmix_quantize_v_page, pnmix_score_prefill,
                   pnmix_score_workspace_bytes,
                   pnmix_v_page_bytes)
from .cache import PNMixLayerCache

__all__ = [
    "PAIRS_ADJACENT", "PAIRS_SPLIT_HALF", "PnmixError", "lib", "make_cfg", "page_jobs",
    "pnmix_cfg", "pnmix_check_cfg", "pnmix_decode_attn", "pnmix_decode_attn_paged",
    "pnmix_decode_plan", "pnmix_decode_splits",
    "pnmix_decode_workspace_bytes", "pnmix_hi_pairs", "pnmix_k_page_bytes", "pnmix_last_error",
    "pnmix_mask_words", "pnmix_quantize_k_page", "pnmix_quantize_v_page", "pnmix_score_prefill",
    "pnmix_score_workspace_bytes", "pnmix_v_page_bytes", "pnmix_append_kv", "pnmix_commit_page",
    "pnmix_append_decode_attn", "pnmix_dequant_k_pages", "pnmix_dequant_v_pages",
    "pnmix_decode_attn_noalloc", "pnmix_noalloc_scratch_bytes", "pnmix_quantize_kv_pages",
    "pnmix_prefill_fused", "pnmix_prefill_fused_workspace_bytes",
    "PNMixLayerCache",
]
