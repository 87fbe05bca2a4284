"""Seeded synthetic inputs for latent-KV decode attention.

This module is the only code shared by the oracle side (tests, bench CPU
baseline) and the GPU side (tests, bench, smoke).  It holds none of the
method's arithmetic: it draws normal variates from numpy's PCG64, rounds
them to bfloat16 (round-to-nearest-even), lays them out in paged caches and
builds block tables.  Nothing here computes a score, a softmax or a
projection.

Workloads mirror the shapes the pages model:
  * the MLA absorbed path at DeepSeek-V3 shape (h_q = 128 heads over a
    latent of 512 plus a shared RoPE key of 64), which reproduces the ~242
    FLOPs/byte the GQLA explainer (technical summary section 2) quotes;
  * the GQLA grouped path (g = 8 groups of d_h = 128, s_q = 2), GQLA
    technical summary sections 2-3;
  * plain GQA vs GLA-2 (two latent heads), the GTA/GLA article's GLA
    section; and a long-context ragged batch (1K-64K, the article's decode
    range);
  * variants on the same kernels: GQLA with g = 4 and s_q = 1, four query
    tokens per step (multi-token prediction), GTA's tied key/value groups
    and GQA-2 with 64 query heads per KV head (VHA's inference form).
Draw order inside one seed: seqlens, block table, q_nope (or q), q_rope,
c_kv (or K then V), k_rope, W_UK, W_UV.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# bfloat16 bit handling (data preparation, not arithmetic of the method)
# --------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        r = (c + (((c >> 16) & 1) + 0x7FFF)) >> 16
        nan = (c & 0x7FFFFFFF) > 0x7F800000
        r = r.astype(np.uint16)
        r[nan] = BF16_NAN
        flat_o[s:s + step] = r
    return out


# OCP 8-bit float E4M3 ("fn": no infinities; S.1111.111 is NaN), the
# positive codes 0x00..0x7E in increasing order of value
E4M3_NAN = np.uint8(0x7F)


def _e4m3_positive_values() -> np.ndarray:
    codes = np.arange(0x7F)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e - 10.0))


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to OCP E4M3 codes: nearest, ties to the even code;
    magnitudes beyond 448 saturate to 448; NaN to 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    vals = _e4m3_positive_values()
    a = np.minimum(np.abs(x), vals[-1])
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, vals.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    code = pick.astype(np.uint8) | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(x), E4M3_NAN, code).astype(np.uint8)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16 bits, generated in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, n, step):
        m = min(step, n - s)
        x = rng.standard_normal(m, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:s + m] = to_bf16_bits(x)
    return out.reshape(shape)


def _normal(rng, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    if dtype == "bf16":
        return _normal_bf16(rng, shape, std)
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _nan_of(dtype: str):
    return BF16_NAN if dtype == "bf16" else np.float32(np.nan)


# --------------------------------------------------------------------------
# sequence lengths and block tables
# --------------------------------------------------------------------------
def log_uniform_seqlens(rng, B: int, lo: int, hi: int) -> np.ndarray:
    """L_b = floor(exp(U(ln lo, ln hi))), clamped to [lo, hi]."""
    u = rng.uniform(math.log(lo), math.log(hi), size=B)
    return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int32)


def make_block_table(rng, seqlens: np.ndarray, page_size: int, max_pages: int | None,
                     kind: str):
    """Block table int32 [B, max_pages], -1 beyond each sequence's pages.

    kind: 'identity'   pages laid out in order;
          'shuffled' / 'random'  a random permutation of an exact-size pool;
          'fragmented' a pool 1.5x the needed pages, a random subset used in
                       random order (the rest stay unused).
    Returns (table, num_pages_in_pool).
    """
    need = [(int(L) + page_size - 1) // page_size for L in seqlens]
    total = sum(need)
    if max_pages is None:
        max_pages = max(need) if need else 1
    if kind == "identity":
        pool = total
        order = np.arange(total)
    elif kind in ("shuffled", "random"):
        pool = total
        order = rng.permutation(total)
    elif kind == "fragmented":
        pool = (3 * total + 1) // 2
        order = rng.permutation(pool)[:total]
    else:
        raise ValueError(kind)
    table = np.full((len(seqlens), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        if n > max_pages:
            raise ValueError("sequence needs more pages than max_pages")
        table[b, :n] = order[pos:pos + n]
        pos += n
    return table, int(pool)


def valid_slot_mask(table: np.ndarray, seqlens: np.ndarray, page_size: int,
                    num_pages: int) -> np.ndarray:
    """bool [num_pages, page_size]: True where a slot holds a valid token."""
    mask = np.zeros((num_pages, page_size), dtype=bool)
    for b, L in enumerate(seqlens):
        L = int(L)
        n = (L + page_size - 1) // page_size
        for i in range(n):
            k = min(page_size, L - i * page_size)
            mask[table[b, i], :k] = True
    return mask


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # 'mla' (latent cache, V = latent) or 'gqa' (expanded K/V)
    dtype: str                # 'bf16' or 'f32'
    B: int
    h_q: int
    s_q: int
    page_size: int
    # mla
    n_lat: int = 1
    d_c: int = 0
    # gqa / gqla
    n_kv: int = 0
    d_h: int = 0
    d_rope: int = 0
    seqlens: tuple = ()
    seqlen_range: tuple = ()  # (lo, hi) log-uniform when seqlens is empty
    table: str = "shuffled"
    max_pages: int | None = None
    causal: bool = True
    # '' = the cache holds the input dtype; 'fp8' = OCP E4M3 codes x8 of
    # values kv_scale * x8 (one scale for the whole cache)
    cache: str = ""
    kv_scale: float = 1.0 / 16
    scale: float = 0.0
    seed: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def softmax_scale(self) -> float:
        return self.scale


def _w(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS = {
    # 1: tiny fp32, oracle in well under a second
    "tiny_mla_fp32": _w(name="tiny_mla_fp32", kind="mla", dtype="f32", B=2, h_q=16, s_q=1,
                        page_size=16, n_lat=1, d_c=64, d_rope=16, seqlens=(200, 256),
                        table="random", scale=1 / math.sqrt(80), seed=1),
    # 2: DeepSeek-V3-shaped MLA absorbed decode (the headline workload)
    "dsv3_mla_b64_l4096": _w(name="dsv3_mla_b64_l4096", kind="mla", dtype="bf16", B=64,
                             h_q=128, s_q=1, page_size=64, n_lat=1, d_c=512, d_rope=64,
                             seqlens=(4096,) * 64, table="shuffled",
                             scale=1 / math.sqrt(576), seed=2),
    # 3: GQLA grouped path from the same weights (latent expanded into 8 groups)
    "gqla_grouped_b64_l4096_sq2": _w(name="gqla_grouped_b64_l4096_sq2", kind="gqla",
                                     dtype="bf16", B=64, h_q=128, s_q=2, page_size=64,
                                     n_lat=1, d_c=512, n_kv=8, d_h=128, d_rope=64,
                                     seqlens=(4096,) * 64, table="shuffled",
                                     scale=1 / math.sqrt(192), seed=3),
    # 4a: plain GQA baseline, 32 q heads over 8 KV heads
    "gqa_b128_l8192": _w(name="gqa_b128_l8192", kind="gqa", dtype="bf16", B=128, h_q=32, s_q=1,
                         page_size=64, n_kv=8, d_h=128, d_rope=0, seqlens=(8192,) * 128,
                         table="shuffled", scale=1 / math.sqrt(128), seed=4),
    # 4b: GLA-2, two latent heads of 256 with 16 q heads each, shared RoPE key
    "gla2_b128_l8192": _w(name="gla2_b128_l8192", kind="mla", dtype="bf16", B=128, h_q=32,
                          s_q=1, page_size=64, n_lat=2, d_c=256, d_rope=64,
                          seqlens=(8192,) * 128, table="shuffled", scale=1 / math.sqrt(320),
                          seed=4),
    # 5: long-context ragged MLA, s_q = 1 and 2
    "ragged_mla_b16_sq1": _w(name="ragged_mla_b16_sq1", kind="mla", dtype="bf16", B=16, h_q=128,
                             s_q=1, page_size=64, n_lat=1, d_c=512, d_rope=64,
                             seqlen_range=(1024, 65536), table="fragmented", max_pages=1024,
                             scale=1 / math.sqrt(576), seed=5),
    "ragged_mla_b16_sq2": _w(name="ragged_mla_b16_sq2", kind="mla", dtype="bf16", B=16, h_q=128,
                             s_q=2, page_size=64, n_lat=1, d_c=512, d_rope=64,
                             seqlen_range=(1024, 65536), table="fragmented", max_pages=1024,
                             scale=1 / math.sqrt(576), seed=5),
    # variants on the same kernels
    # GQLA grouped path with g = 4 groups and one query token (the GQLA
    # explainer's other grouped setting)
    "gqla_g4_b64_l4096_sq1": _w(name="gqla_g4_b64_l4096_sq1", kind="gqla", dtype="bf16", B=64,
                                h_q=128, s_q=1, page_size=64, n_lat=1, d_c=512, n_kv=4, d_h=128,
                                d_rope=64, seqlens=(4096,) * 64, table="shuffled",
                                scale=1 / math.sqrt(192), seed=6),
    # multi-token prediction: four query tokens per step on the MLA path
    "mtp_mla_b64_l4096_sq4": _w(name="mtp_mla_b64_l4096_sq4", kind="mla", dtype="bf16", B=64,
                                h_q=128, s_q=4, page_size=64, n_lat=1, d_c=512, d_rope=64,
                                seqlens=(4096,) * 64, table="shuffled",
                                scale=1 / math.sqrt(576), seed=7),
    # GTA (grouped-tied attention): 8 groups whose key and value are one
    # tied 128-wide state, plus a shared 64-wide RoPE key -- the absorbed
    # layout with one latent head per group
    "gta_b128_l8192": _w(name="gta_b128_l8192", kind="mla", dtype="bf16", B=128, h_q=32, s_q=1,
                         page_size=64, n_lat=8, d_c=128, d_rope=64, seqlens=(8192,) * 128,
                         table="shuffled", scale=1 / math.sqrt(192), seed=8),
    # GQA-2 (two KV heads, 64 query heads each), the inference form of VHA
    "vha_gqa2_b64_l8192": _w(name="vha_gqa2_b64_l8192", kind="gqa", dtype="bf16", B=64, h_q=128,
                             s_q=1, page_size=64, n_kv=2, d_h=128, d_rope=0,
                             seqlens=(8192,) * 64, table="shuffled", scale=1 / math.sqrt(128),
                             seed=9),
}
# 8-bit (OCP E4M3) caches of the same draws, one scale per cache
for _n in ("dsv3_mla_b64_l4096", "gla2_b128_l8192", "gqa_b128_l8192"):
    WORKLOADS[_n + "_fp8"] = replace(WORKLOADS[_n], name=_n + "_fp8", cache="fp8")


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _seqlens(rng, w: Workload) -> np.ndarray:
    if w.seqlens:
        return np.asarray(w.seqlens, dtype=np.int32)
    lo, hi = w.seqlen_range
    return log_uniform_seqlens(rng, w.B, lo, hi)


def generate(w: Workload, *, poison: bool = True, seqlens=None) -> dict:
    """Draw every input of workload ``w`` from PCG64(w.seed).

    Returns a dict of numpy arrays (bf16 as uint16 bits, f32 as float32):
      seqlens [B], block_table [B, max_pages], num_pages,
      mla/gqla: kv [num_pages, page_size, n_lat*d_c + d_rope] packed cache
                (c_kv = kv[..., :n_lat*d_c], k_rope = kv[..., n_lat*d_c:]),
                q_nope [B, s_q, h_q, d_c] (absorbed query; for 'gqla' the
                un-absorbed q [B, s_q, h_q, d_h] is q_nope_h), q_rope,
                gqla also w_uk, w_uv [g, d_c, d_h] ~ N(0, 1/d_c);
      gqa:      q [B, s_q, h_q, d_h], k_cache, v_cache [num_pages,
                page_size, n_kv, d_h].
    Slots that hold no valid token are NaN when ``poison`` is set.
    """
    rng = np.random.default_rng(w.seed)
    sl = np.asarray(seqlens, dtype=np.int32) if seqlens is not None else _seqlens(rng, w)
    table, num_pages = make_block_table(rng, sl, w.page_size, w.max_pages, w.table)
    out = {"seqlens": sl, "block_table": table, "num_pages": num_pages}
    P, dt = w.page_size, w.dtype
    if w.kind in ("mla", "gqla"):
        width = w.n_lat * w.d_c + w.d_rope
        if w.kind == "gqla":
            out["q_nope_h"] = _normal(rng, (w.B, w.s_q, w.h_q, w.d_h), dt)
        else:
            out["q_nope"] = _normal(rng, (w.B, w.s_q, w.h_q, w.d_c), dt)
        out["q_rope"] = _normal(rng, (w.B, w.s_q, w.h_q, w.d_rope), dt)
        kv = np.empty((num_pages, P, width), dtype=np.uint16 if dt == "bf16" else np.float32)
        kv[..., :w.n_lat * w.d_c] = _normal(rng, (num_pages, P, w.n_lat * w.d_c), dt)
        kv[..., w.n_lat * w.d_c:] = _normal(rng, (num_pages, P, w.d_rope), dt)
        out["kv"] = kv
        if w.kind == "gqla":
            std = 1.0 / math.sqrt(w.d_c)
            out["w_uk"] = _normal(rng, (w.n_kv, w.d_c, w.d_h), dt, std)
            out["w_uv"] = _normal(rng, (w.n_kv, w.d_c, w.d_h), dt, std)
        caches = [kv]
    elif w.kind == "gqa":
        out["q"] = _normal(rng, (w.B, w.s_q, w.h_q, w.d_h), dt)
        if w.d_rope:
            out["q_rope"] = _normal(rng, (w.B, w.s_q, w.h_q, w.d_rope), dt)
        out["k_cache"] = _normal(rng, (num_pages, P, w.n_kv, w.d_h), dt)
        out["v_cache"] = _normal(rng, (num_pages, P, w.n_kv, w.d_h), dt)
        caches = [out["k_cache"], out["v_cache"]]
        if w.d_rope:
            out["k_rope"] = _normal(rng, (num_pages, P, w.d_rope), dt)
            caches.append(out["k_rope"])
    else:
        raise ValueError(w.kind)
    if poison:
        invalid = ~valid_slot_mask(table, sl, P, num_pages)
        for c in caches:
            c[invalid] = _nan_of(dt)
    if w.cache == "fp8":
        # the same draws, stored as E4M3 codes of value / kv_scale
        keys = ["kv"] if w.kind in ("mla", "gqla") else ["k_cache", "v_cache"] + (
            ["k_rope"] if w.d_rope else [])
        if dt == "bf16":
            # every bf16 pattern through the encoder once, then a lookup
            allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
            with np.errstate(invalid="ignore"):  # signalling-NaN patterns
                lut = to_e4m3_bits(bf16_bits_to_f32(allbits).astype(np.float64) / w.kv_scale)
        for k in keys:
            if dt == "bf16":
                out[k] = lut[out[k]]
            else:
                out[k] = to_e4m3_bits(out[k].astype(np.float64) / w.kv_scale)
        out["kv_scale"] = w.kv_scale
    return out


def sample_rows(rng_seed: int, B: int, s_q: int, h_q: int, n: int) -> np.ndarray:
    """Flat row ids (b*s_q + t)*h_q + h for a seeded sample that always
    includes the first and the last row."""
    total = B * s_q * h_q
    rng = np.random.default_rng(rng_seed)
    pick = rng.choice(total, size=min(n, total), replace=False)
    pick = np.unique(np.concatenate([pick, [0, total - 1]])).astype(np.int32)
    return pick
