"""Roofline arithmetic for decode attention over a compressed KV cache.

Algorithmic work is what the method must move or compute, independent of how
a kernel does it:
  bytes  = every visible cache token read once (latent + shared RoPE key, or
           expanded K/V + RoPE key), plus query, output, LSE, block-table
           entries of used pages and the lengths;
  FLOPs  = per visible (query row, cache token) pair: 2*(key width) for the
           score and 2*(value width) for the weighted sum (exponentials are
           not counted).
Per-token figures follow the GQLA explainer (technical summary sections 2
and 4): the MQA-absorbed path keeps r_kv + d^R_h elements per token and does
h_q*(2*(d_c + d_rope) + 2*d_c) FLOPs per cache token per query token; the GQA
path keeps 2*g*d_h + d^R_h elements per token.  An 8-bit cache (cache_elem =
1) halves the cache bytes; query and output stay 2 bytes per element.
"""
from __future__ import annotations

from dataclasses import dataclass

# MI355X published peaks (dense, no sparsity).
MI355X_HBM_GBPS = 8000.0
MI355X_BF16_TFLOPS = 2500.0
MI355X_FP8_TFLOPS = 5000.0
MI355X_FP32_TFLOPS = 157.3


def ridge(peak_flops: float, bandwidth_bytes: float) -> float:
    """FLOPs per byte at which a roofline turns from memory- to compute-bound."""
    return peak_flops / bandwidth_bytes


def absorbed_intensity(h_q: int, d_c: int, d_rope: int, s_q: int = 1, elem: int = 2) -> float:
    """Cache-only arithmetic intensity of the MQA-absorbed path: FLOPs per
    cache byte (every query token of the step reuses the same cache read)."""
    return s_q * h_q * (2 * (d_c + d_rope) + 2 * d_c) / ((d_c + d_rope) * elem)


def grouped_intensity(h_q: int, g: int, d_h: int, d_rope: int, s_q: int = 1, elem: int = 2) -> float:
    """Cache-only arithmetic intensity of the GQA path over the expanded cache."""
    return s_q * h_q * (2 * (d_h + d_rope) + 2 * d_h) / ((2 * g * d_h + d_rope) * elem)


def kv_ratio(d_c: int, d_rope: int, g: int, d_h: int) -> float:
    """Per-token cache of the absorbed path relative to a GQA baseline with g
    KV heads of width d_h (K and V, no RoPE key)."""
    return (d_c + d_rope) / (2 * g * d_h)


def decode_tokens_per_s(peak_flops: float, bandwidth: float, cache_tokens: int, *,
                        bytes_per_cache_token: float, flops_per_cache_token_per_query: float,
                        s_q: int = 1) -> float:
    """One-layer roofline throughput: each step reads `cache_tokens` tokens once
    and serves s_q query tokens."""
    t_mem = cache_tokens * bytes_per_cache_token / bandwidth
    t_cmp = s_q * cache_tokens * flops_per_cache_token_per_query / peak_flops
    return s_q / max(t_mem, t_cmp)


@dataclass
class Work:
    bytes: float
    flops: float
    cache_bytes: float

    @property
    def intensity(self) -> float:
        return self.flops / self.bytes


def _visible(L: int, s_q: int, t: int, causal: bool) -> int:
    return max(0, L - s_q + t + 1) if causal else max(0, L)


def mla_work(seqlens, *, s_q: int, h_q: int, n_lat: int, d_c: int, d_rope: int, page_size: int,
             causal: bool = True, elem: int = 2, cache_elem: int | None = None) -> Work:
    tok = sum(int(L) for L in seqlens)
    cache = tok * (n_lat * d_c + d_rope) * (elem if cache_elem is None else cache_elem)
    B = len(seqlens)
    rows = B * s_q * h_q
    q = rows * (d_c + d_rope) * elem
    out = rows * d_c * elem + rows * 4
    pages = sum((int(L) + page_size - 1) // page_size for L in seqlens)
    meta = pages * 4 + B * 4
    pairs = sum(_visible(int(L), s_q, t, causal) for L in seqlens for t in range(s_q))
    flops = pairs * h_q * (2 * (d_c + d_rope) + 2 * d_c)
    return Work(bytes=cache + q + out + meta, flops=flops, cache_bytes=cache)


def gqa_work(seqlens, *, s_q: int, h_q: int, n_kv: int, d_h: int, d_rope: int, page_size: int,
             causal: bool = True, elem: int = 2, cache_elem: int | None = None) -> Work:
    tok = sum(int(L) for L in seqlens)
    cache = tok * (2 * n_kv * d_h + d_rope) * (elem if cache_elem is None else cache_elem)
    B = len(seqlens)
    rows = B * s_q * h_q
    q = rows * (d_h + d_rope) * elem
    out = rows * d_h * elem + rows * 4
    pages = sum((int(L) + page_size - 1) // page_size for L in seqlens)
    meta = pages * 4 + B * 4
    pairs = sum(_visible(int(L), s_q, t, causal) for L in seqlens for t in range(s_q))
    flops = pairs * h_q * (2 * (d_h + d_rope) + 2 * d_h)
    return Work(bytes=cache + q + out + meta, flops=flops, cache_bytes=cache)


def expand_work(n_tokens: int, *, g: int, d_c: int, d_h: int, elem: int = 2,
                out_elem: int | None = None) -> Work:
    """Latent expansion at cache-write time: read the latent once, write 2g
    groups of d_h (out_elem bytes each: 1 for an 8-bit cache), 2 FLOPs per
    multiply-add."""
    rd = n_tokens * d_c * elem + 2 * g * d_c * d_h * elem
    wr = n_tokens * 2 * g * d_h * (elem if out_elem is None else out_elem)
    return Work(bytes=rd + wr, flops=2.0 * n_tokens * d_c * 2 * g * d_h, cache_bytes=rd)
