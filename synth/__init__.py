"""Seeded synthetic inputs for the PN-Mix key-cache path.

This module holds none of the method's arithmetic: it only draws post-RoPE queries and keys
and values of the shapes and value structure the pages' workloads have, so that the HIP path
and the CPU oracle can be fed the same fp16 bits.

Recipe (one draw per (workload, layer, tensor, chunk) stream, base seed 42):
  * per-(head, RoPE pair) scales a = exp(sigma_ln * N(0, 1)), drawn once per head for Q and
    independently for K, shared by every batch row and token: persistent outlier pairs, the
    structure the PN-Mix paper's sec. 4 and the KV-quantization blog's "Keys and values are
    not the same tensor" section describe for post-RoPE keys;
  * each token's pair (u, v) ~ N(0, 1)^2 is scaled by a and rotated by the angle t * theta_i,
    theta_i = base^(-2i/d), with the configured pairing (adjacent (2i, 2i+1) or split-half
    (i, i + d/2)); the arithmetic is fp32 and the result is rounded to fp16 (round half even);
  * values V ~ N(0, 1) in fp16;
  * the decode query of a step at position t uses the same law as prefill queries.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import torch

BASE_SEED = 42


def derive_seed(*parts) -> int:
    """Stable 63-bit seed from the base seed and a tuple of labels."""
    h = hashlib.sha256("/".join(str(p) for p in (BASE_SEED,) + parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(*parts))
    return g


def pair_scales(n_heads: int, n_pairs: int, sigma_ln: float, device, *seed_parts) -> torch.Tensor:
    """exp(sigma_ln * N(0,1)) per (head, pair), float32 [n_heads][n_pairs]."""
    g = _gen(device, "scales", *seed_parts)
    z = torch.randn(n_heads, n_pairs, generator=g, device=device, dtype=torch.float32)
    return torch.exp(sigma_ln * z)


def rope_tokens(scales: torch.Tensor, batch: int, positions: torch.Tensor, d: int, pairing: int,
                base: float, device, *seed_parts) -> torch.Tensor:
    """Post-RoPE fp16 tokens [batch][heads][len(positions)][d] with pair scales `scales`."""
    H, npairs = scales.shape
    assert npairs == d // 2
    T = positions.numel()
    g = _gen(device, "tok", *seed_parts)
    uv = torch.randn(batch, H, T, npairs, 2, generator=g, device=device, dtype=torch.float32)
    uv = uv * scales.view(1, H, 1, npairs, 1)
    i = torch.arange(npairs, device=device, dtype=torch.float32)
    theta = torch.pow(torch.tensor(float(base), device=device, dtype=torch.float32),
                      -2.0 * i / float(d))
    ang = positions.to(device=device, dtype=torch.float32).view(T, 1) * theta.view(1, npairs)
    cs, sn = torch.cos(ang), torch.sin(ang)
    u, v = uv[..., 0], uv[..., 1]
    x = u * cs - v * sn
    y = u * sn + v * cs
    out = torch.empty(batch, H, T, d, device=device, dtype=torch.float32)
    if pairing == 0:
        out[..., 0::2] = x
        out[..., 1::2] = y
    else:
        out[..., : d // 2] = x
        out[..., d // 2:] = y
    return out.to(torch.float16)


def values(batch: int, heads: int, T: int, d: int, device, *seed_parts) -> torch.Tensor:
    g = _gen(device, "val", *seed_parts)
    return torch.randn(batch, heads, T, d, generator=g, device=device,
                       dtype=torch.float32).to(torch.float16)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: model shape, PN-Mix settings and cache length."""
    name: str
    layers: int
    B: int
    H_q: int
    H_kv: int
    d: int
    pairing: int           # 0 adjacent, 1 split-half
    rope_base: float
    P: int                 # prefill length
    T: int                 # cached tokens at the measured decode step
    r: float
    G: int
    b_V: int = 2
    g_V: int = 32
    b_H: int = 3
    b_L: int = 1
    N_s: int = 32
    N: int = 128
    sigma_ln: float = 1.0
    prefill_score_P: int = 0   # extra long-prefill scoring pass (B = 1), 0 if none

    @property
    def n_hi_pairs(self) -> int:
        return int(math.floor(self.r * (self.d // 2) + 1e-9))

    @property
    def n_pages(self) -> int:
        return (self.T - self.N_s) // self.N

    @property
    def res_len(self) -> int:
        return self.T - self.N_s - self.n_pages * self.N


# The five workloads of the PN-Mix key-cache path, in order: a tiny one the oracle runs in
# seconds, then shapes of Qwen3-8B (one layer at 32K; 36 layers at B=32, 8K), Llama-3.1-8B
# (B=110, 8K, PN-Mix(2), plus a 16K prefill score) and Qwen3-32B (64/8 heads, B=32, 32K).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 4, 2, 32, 0, 1e4, 64, 512, 0.5, 128, sigma_ln=1.0),
    "qwen3-8b-1L-32k": Workload("qwen3-8b-1L-32k", 1, 1, 32, 8, 128, 1, 1e6, 141, 32768, 0.5,
                                128),
    "qwen3-8b-36L-b32-8k": Workload("qwen3-8b-36L-b32-8k", 36, 32, 32, 8, 128, 1, 1e6, 141,
                                    8192, 0.5, 128),
    "llama3.1-8b-32L-b110-8k": Workload("llama3.1-8b-32L-b110-8k", 32, 110, 32, 8, 128, 1, 5e5,
                                        141, 8192, 0.4, 64, prefill_score_P=16384),
    "qwen3-32b-64L-b32-32k": Workload("qwen3-32b-64L-b32-32k", 64, 32, 64, 8, 128, 1, 1e6, 141,
                                      32768, 0.5, 128, sigma_ln=1.5),
}
