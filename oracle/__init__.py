"""fp64 CPU oracle for latent-KV decode attention (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never imports it, and it imports nothing
from the product path.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
rows).  This module only builds that file with gcc and marshals numpy arrays
into it.  Each wrapper names the passage of the pages it follows; the C
source states the same definitions.

Pins: every function here is pinned by ``tests/test_oracle.py`` against
something other than itself (a library attention routine on gathered
inputs, closed forms, the absorb identity, the copy special case, split
invariance).  No function is parity-unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# LKV_ORACLE_SANITIZE=1: build and load an AddressSanitizer + UBSan build of
# the oracle instead (for CPU tests run with the sanitizer runtime preloaded)
SANITIZE = os.environ.get("LKV_ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liblkv_oracle_san.so" if SANITIZE else "liblkv_oracle.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"]

F32, BF16, F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c into liblkv_oracle.so (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             *(_SAN_FLAGS if SANITIZE else []), "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        _lib.oracle_mla_decode.restype = ctypes.c_int
        _lib.oracle_gqa_decode.restype = ctypes.c_int
        _lib.oracle_mla_explicit.restype = ctypes.c_int
        _lib.oracle_expand_latent.restype = ctypes.c_int
        _lib.oracle_mla_row_weights.restype = ctypes.c_int
        _lib.oracle_num_threads.restype = ctypes.c_int
    return _lib


_P = ctypes.c_void_p


class _MlaArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("s_q", ctypes.c_int), ("h_q", ctypes.c_int),
                ("n_lat", ctypes.c_int), ("d_c", ctypes.c_int), ("d_rope", ctypes.c_int),
                ("page_size", ctypes.c_int), ("max_pages", ctypes.c_int),
                ("scale", ctypes.c_double), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
                ("q_nope", _P), ("q_rope", _P), ("c_kv", _P), ("kv_tok_stride", ctypes.c_longlong),
                ("k_rope", _P), ("rope_tok_stride", ctypes.c_longlong),
                ("block_table", _P), ("seqlens", _P), ("range_lo", _P), ("range_hi", _P),
                ("rows", _P), ("n_rows", ctypes.c_longlong), ("out", _P), ("lse", _P)]


class _GqaArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("s_q", ctypes.c_int), ("h_q", ctypes.c_int),
                ("n_kv", ctypes.c_int), ("d_h", ctypes.c_int), ("d_rope", ctypes.c_int),
                ("page_size", ctypes.c_int), ("max_pages", ctypes.c_int),
                ("scale", ctypes.c_double), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
                ("q", _P), ("q_rope", _P), ("k_cache", _P), ("k_tok_stride", ctypes.c_longlong),
                ("v_cache", _P), ("v_tok_stride", ctypes.c_longlong),
                ("k_rope", _P), ("rope_tok_stride", ctypes.c_longlong),
                ("block_table", _P), ("seqlens", _P), ("rows", _P), ("n_rows", ctypes.c_longlong),
                ("out", _P), ("lse", _P)]


class _ExplicitArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("s_q", ctypes.c_int), ("h_q", ctypes.c_int),
                ("n_w", ctypes.c_int), ("d_c", ctypes.c_int), ("d_h", ctypes.c_int),
                ("d_rope", ctypes.c_int), ("page_size", ctypes.c_int), ("max_pages", ctypes.c_int),
                ("scale", ctypes.c_double), ("causal", ctypes.c_int), ("dtype", ctypes.c_int),
                ("q_nope", _P), ("q_rope", _P), ("w_uk", _P), ("w_uv", _P),
                ("c_kv", _P), ("kv_tok_stride", ctypes.c_longlong),
                ("k_rope", _P), ("rope_tok_stride", ctypes.c_longlong),
                ("block_table", _P), ("seqlens", _P), ("out", _P), ("lse", _P)]


class _ExpandArgs(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("g", ctypes.c_int), ("d_c", ctypes.c_int),
                ("d_h", ctypes.c_int), ("page_size", ctypes.c_int), ("max_pages", ctypes.c_int),
                ("dtype", ctypes.c_int), ("c_kv", _P), ("kv_tok_stride", ctypes.c_longlong),
                ("w_uk", _P), ("w_uv", _P), ("block_table", _P), ("seqlens", _P),
                ("start_pos", _P), ("k_out", _P), ("v_out", _P)]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cache_dtype(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"arrays must be float32, uint16 (bf16 bits) or float64, got {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops for later calls (timing
    only; the arithmetic and its order per row do not depend on it)."""
    _load().oracle_set_num_threads(ctypes.c_int(int(n)))


def mla_decode(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, *, n_lat, d_c, d_rope,
               page_size, scale, causal=True, kv_tok_stride=None, rope_tok_stride=None,
               range_lo=None, range_hi=None, rows=None):
    """O1 -- MLA absorbed decode (GQLA technical summary section 2, MQA-absorbed
    path; GLA section for several latent heads).

    q_nope [B, s_q, h_q, d_c], q_rope [B, s_q, h_q, d_rope]: absorbed query,
    float32 or bf16 bits (uint16).  c_kv / k_rope: flat paged caches (any
    shape; only the element offsets matter), same dtype.  Returns
    (out float64 [B, s_q, h_q, d_c], lse float64 [B, s_q, h_q]).  With
    ``rows`` (flat row ids), only those rows are computed; the rest are NaN.
    """
    q_nope, q_rope = _c(q_nope), _c(q_rope)
    c_kv, k_rope = _c(c_kv), _c(k_rope)
    B, s_q, h_q, dc = q_nope.shape
    assert dc == d_c and q_rope.shape == (B, s_q, h_q, d_rope)
    dt = _cache_dtype(q_nope)
    assert _cache_dtype(c_kv) == dt and _cache_dtype(k_rope) == dt and _cache_dtype(q_rope) == dt
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    lo = _c(range_lo, np.int32)
    hi = _c(range_hi, np.int32)
    rws = _c(rows, np.int32)
    out = np.full((B, s_q, h_q, d_c), np.nan)
    lse = np.full((B, s_q, h_q), np.nan)
    a = _MlaArgs(B, s_q, h_q, n_lat, d_c, d_rope, page_size, bt.shape[1], float(scale),
                 int(bool(causal)), dt, _ptr(q_nope), _ptr(q_rope), _ptr(c_kv),
                 kv_tok_stride if kv_tok_stride is not None else n_lat * d_c,
                 _ptr(k_rope), rope_tok_stride if rope_tok_stride is not None else d_rope,
                 _ptr(bt), _ptr(sl), _ptr(lo), _ptr(hi), _ptr(rws),
                 0 if rws is None else rws.size, _ptr(out), _ptr(lse))
    rc = _load().oracle_mla_decode(ctypes.byref(a))
    if rc:
        raise RuntimeError(f"oracle_mla_decode failed ({rc})")
    return out, lse


def mla_row_weights(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, b, t, h, *, n_lat,
                    d_c, d_rope, page_size, scale, causal=True, kv_tok_stride=None,
                    rope_tok_stride=None):
    """Softmax weights of one O1 row, for the normalisation pin."""
    q_nope, q_rope = _c(q_nope), _c(q_rope)
    c_kv, k_rope = _c(c_kv), _c(k_rope)
    B, s_q, h_q, _ = q_nope.shape
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    cap = int(sl.max()) + 1
    p = np.zeros(cap)
    a = _MlaArgs(B, s_q, h_q, n_lat, d_c, d_rope, page_size, bt.shape[1], float(scale),
                 int(bool(causal)), _cache_dtype(q_nope), _ptr(q_nope), _ptr(q_rope), _ptr(c_kv),
                 kv_tok_stride if kv_tok_stride is not None else n_lat * d_c,
                 _ptr(k_rope), rope_tok_stride if rope_tok_stride is not None else d_rope,
                 _ptr(bt), _ptr(sl), None, None, None, 0, None, None)
    n = _load().oracle_mla_row_weights(ctypes.byref(a), int(b), int(t), int(h), _ptr(p), cap)
    if n < 0:
        raise RuntimeError("oracle_mla_row_weights failed")
    return p[:n]


def gqa_decode(q, k_cache, v_cache, block_table, seqlens, *, n_kv, d_h, page_size, scale,
               causal=True, q_rope=None, k_rope=None, d_rope=0, k_tok_stride=None,
               v_tok_stride=None, rope_tok_stride=None, rows=None):
    """O3 -- grouped-query decode over an expanded cache (GQLA technical
    summary section 2, GQA path; plain GQA when there is no RoPE key).

    q [B, s_q, h_q, d_h]; k_cache / v_cache paged with element (p, s, g, d) at
    (p*page_size + s)*tok_stride + g*d_h + d; optional shared k_rope.
    Returns (out float64 [B, s_q, h_q, d_h], lse float64 [B, s_q, h_q]).
    """
    q = _c(q)
    k_cache, v_cache = _c(k_cache), _c(v_cache)
    q_rope, k_rope = _c(q_rope), _c(k_rope)
    B, s_q, h_q, dh = q.shape
    assert dh == d_h
    dt = _cache_dtype(q)
    assert _cache_dtype(k_cache) == dt and _cache_dtype(v_cache) == dt
    if d_rope:
        assert q_rope.shape == (B, s_q, h_q, d_rope) and _cache_dtype(k_rope) == dt
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    rws = _c(rows, np.int32)
    out = np.full((B, s_q, h_q, d_h), np.nan)
    lse = np.full((B, s_q, h_q), np.nan)
    a = _GqaArgs(B, s_q, h_q, n_kv, d_h, d_rope, page_size, bt.shape[1], float(scale),
                 int(bool(causal)), dt, _ptr(q), _ptr(q_rope) if d_rope else None, _ptr(k_cache),
                 k_tok_stride if k_tok_stride is not None else n_kv * d_h, _ptr(v_cache),
                 v_tok_stride if v_tok_stride is not None else n_kv * d_h,
                 _ptr(k_rope) if d_rope else None,
                 rope_tok_stride if rope_tok_stride is not None else d_rope,
                 _ptr(bt), _ptr(sl), _ptr(rws), 0 if rws is None else rws.size,
                 _ptr(out), _ptr(lse))
    rc = _load().oracle_gqa_decode(ctypes.byref(a))
    if rc:
        raise RuntimeError(f"oracle_gqa_decode failed ({rc})")
    return out, lse


def mla_explicit(q_nope_h, q_rope, w_uk, w_uv, c_kv, k_rope, block_table, seqlens, *, page_size,
                 scale, causal=True, kv_tok_stride=None, rope_tok_stride=None):
    """O2 -- explicit (non-absorbed) MLA / GQLA decode (X post: per-head
    mixing of the latent; GQLA technical summary section 2: group-indexed
    W_UK, W_UV).  q_nope_h [B, s_q, h_q, d_h] is the un-absorbed query
    (float64); w_uk, w_uv [n_w, d_c, d_h] float64.  Returns (o [B, s_q, h_q,
    d_h], lse)."""
    q_nope_h = _c(q_nope_h, np.float64)
    q_rope = _c(q_rope, np.float64)
    w_uk, w_uv = _c(w_uk, np.float64), _c(w_uv, np.float64)
    c_kv, k_rope = _c(c_kv), _c(k_rope)
    B, s_q, h_q, d_h = q_nope_h.shape
    n_w, d_c, dh2 = w_uk.shape
    assert dh2 == d_h and w_uv.shape == w_uk.shape
    d_rope = q_rope.shape[-1]
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    out = np.full((B, s_q, h_q, d_h), np.nan)
    lse = np.full((B, s_q, h_q), np.nan)
    a = _ExplicitArgs(B, s_q, h_q, n_w, d_c, d_h, d_rope, page_size, bt.shape[1], float(scale),
                      int(bool(causal)), _cache_dtype(c_kv), _ptr(q_nope_h), _ptr(q_rope),
                      _ptr(w_uk), _ptr(w_uv), _ptr(c_kv),
                      kv_tok_stride if kv_tok_stride is not None else d_c, _ptr(k_rope),
                      rope_tok_stride if rope_tok_stride is not None else d_rope,
                      _ptr(bt), _ptr(sl), _ptr(out), _ptr(lse))
    rc = _load().oracle_mla_explicit(ctypes.byref(a))
    if rc:
        raise RuntimeError(f"oracle_mla_explicit failed ({rc})")
    return out, lse


def absorb_query(q_nope_h, w_uk):
    """q'_h = W_UK[w(h)] q_nope_h (GQLA section 2: W_UK folds into the query
    projection).  q_nope_h [B, s_q, h_q, d_h] -> [B, s_q, h_q, d_c] float64."""
    q = _c(q_nope_h, np.float64)
    w = _c(w_uk, np.float64)
    B, s_q, h_q, d_h = q.shape
    n_w, d_c, _ = w.shape
    out = np.empty((B, s_q, h_q, d_c))
    _load().oracle_absorb_query(ctypes.c_longlong(q.size // d_h), h_q, n_w, d_c, d_h,
                                _ptr(q), _ptr(w), _ptr(out))
    return out


def up_project(o_latent, w_uv):
    """o_h = O'_h W_UV[w(h)] (GQLA section 2: W_UV folds into the output
    projection).  o_latent [B, s_q, h_q, d_c] -> [B, s_q, h_q, d_h]."""
    o = _c(o_latent, np.float64)
    w = _c(w_uv, np.float64)
    B, s_q, h_q, d_c = o.shape
    n_w, _, d_h = w.shape
    out = np.empty((B, s_q, h_q, d_h))
    _load().oracle_up_project(ctypes.c_longlong(o.size // d_c), h_q, n_w, d_c, d_h,
                              _ptr(o), _ptr(w), _ptr(out))
    return out


def expand_latent(c_kv, w_uk, w_uv, block_table, seqlens, *, page_size, num_pages,
                  kv_tok_stride=None, start_pos=None):
    """O5 -- latent expansion at cache-write time (GQLA section 2, GQA path).
    Returns (k, v) float64 [num_pages, page_size, g, d_h]; rows of tokens
    that are not expanded hold NaN."""
    c_kv = _c(c_kv)
    w_uk, w_uv = _c(w_uk, np.float64), _c(w_uv, np.float64)
    g, d_c, d_h = w_uk.shape
    bt = _c(block_table, np.int32)
    sl = _c(seqlens, np.int32)
    sp = _c(start_pos, np.int32)
    k = np.full((num_pages, page_size, g, d_h), np.nan)
    v = np.full((num_pages, page_size, g, d_h), np.nan)
    a = _ExpandArgs(bt.shape[0], g, d_c, d_h, page_size, bt.shape[1], _cache_dtype(c_kv),
                    _ptr(c_kv), kv_tok_stride if kv_tok_stride is not None else d_c,
                    _ptr(w_uk), _ptr(w_uv), _ptr(bt), _ptr(sl), _ptr(sp), _ptr(k), _ptr(v))
    _load().oracle_expand_latent(ctypes.byref(a))
    return k, v


def lse_combine(o_part, lse_part, work_offsets):
    """O4 combine -- merge split-KV partials (the LSE-weighted merge).
    o_part [n_work, s_q, h_q, d_v], lse_part [n_work, s_q, h_q],
    work_offsets [B+1].  Returns (out [B, s_q, h_q, d_v], lse [B, s_q, h_q])."""
    o = _c(o_part, np.float64)
    l = _c(lse_part, np.float64)
    off = _c(work_offsets, np.int32)
    _, s_q, h_q, d_v = o.shape
    B = off.size - 1
    out = np.empty((B, s_q, h_q, d_v))
    lse = np.empty((B, s_q, h_q))
    _load().oracle_lse_combine(B, s_q, h_q, d_v, _ptr(o), _ptr(l), _ptr(off), _ptr(out), _ptr(lse))
    return out, lse


def append_tokens(src, cache, block_table, seqlens, *, page_size, tok_stride):
    """Cache write of a step's new tokens (GQLA section 2: every token's latent
    and the shared RoPE key are cached once, per page slot).  Row t of
    sequence b's s_q new rows goes to logical position j = seqlens[b] - s_q +
    t (skipped when j < 0), physical row block_table[b][j // page_size] *
    page_size + j % page_size.  Pure data movement, written out here with
    plain loops.  Returns a flat copy of ``cache`` with those rows written."""
    out = np.array(cache, copy=True).reshape(-1)
    src = np.asarray(src)
    B, s_q, width = src.shape
    for b in range(B):
        for t in range(s_q):
            j = int(seqlens[b]) - s_q + t
            if j < 0:
                continue
            row = int(block_table[b, j // page_size]) * page_size + j % page_size
            out[row * tok_stride: row * tok_stride + width] = src[b, t]
    return out



def e4m3_to_f64(codes, scale=1.0):
    """Values of OCP 8-bit float E4M3 codes times ``scale`` (the "fn" variant:
    sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    holds the subnormals m * 2^-9; S.1111.111 is NaN; no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    v = np.where(s == 1, -mag, mag)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return v * scale


def e4m3_from_f64(x):
    """Nearest OCP E4M3 code of each value: ties go to the even code,
    magnitudes past the largest (448) saturate to it, NaN gives S.1111.111;
    the sign is bit 7 (so -0.0 gives 0x80).  Searches the magnitudes that
    e4m3_to_f64 assigns to codes 0x00..0x7E (increasing)."""
    x = np.asarray(x, dtype=np.float64)
    mags = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), mags[-1])
    hi = np.clip(np.searchsorted(mags, np.nan_to_num(a)), 0, mags.size - 1)
    lo = np.maximum(hi - 1, 0)
    below, above = a - mags[lo], mags[hi] - a
    code = np.where(below < above, lo, np.where(above < below, hi, np.where(lo % 2 == 0, lo, hi)))
    code = code.astype(np.uint8) | np.where(np.signbit(x), np.uint8(0x80), np.uint8(0))
    return np.where(np.isnan(x), np.uint8(0x7F) | code & np.uint8(0x80), code).astype(np.uint8)
