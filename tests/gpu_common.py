"""Shared helpers for the GPU parity tests: move seeded numpy inputs to the
device, call the HIP library through the C ABI binding, and compare with the
oracle under the stated tolerances.

Tolerances (bf16 inputs, fp32 accumulation): output max-abs 2e-2 and
relative L2 5e-3; LSE max-abs 1e-3 (LSE has no stated bound: 1e-3 is about
ten bf16 ulps of P's rounding felt through the log-sum); worst single row
relative L2 1e-2.  float32 path: 1e-5 relative L2, 1e-4 max-abs, 1e-4 per
row.
"""
import math
import sys

import numpy as np

import lkv_inputs as li

OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3
# bound on the worst single output row's relative L2 error (rows with a
# nonzero reference): twice the whole-output bound, so that one bad row (a
# wrong page, a missed rescale) fails even when the rest of the output hides
# it; float32 path 1e-4
ROW_REL_L2 = 1e-2
ROW_REL_L2_F32 = 1e-4


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def from_dev(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def assert_close(out, ref, lse=None, lse_ref=None, *, f32=False, what=""):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    ma = float(np.abs(out - ref).max()) if out.size else 0.0
    rl = rel_l2(out, ref) if out.size else 0.0
    lim_ma, lim_rl = (1e-4, 1e-5) if f32 else (OUT_MAX_ABS, OUT_REL_L2)
    # worst per-row relative L2 (rows with a nonzero reference), reported
    # beside the bound on the whole output
    rows_o = out.reshape(-1, out.shape[-1]) if out.ndim > 1 else out.reshape(1, -1)
    rows_r = ref.reshape(rows_o.shape)
    nr = np.linalg.norm(rows_r, axis=1)
    live = nr > 0
    worst = float((np.linalg.norm(rows_o - rows_r, axis=1)[live] / nr[live]).max()) if live.any() else 0.0
    note(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e} worst_row_rel_l2={worst:.3e}")
    assert ma <= lim_ma, f"{what}: max abs error {ma} > {lim_ma}"
    assert rl <= lim_rl, f"{what}: relative L2 error {rl} > {lim_rl}"
    lim_row = ROW_REL_L2_F32 if f32 else ROW_REL_L2
    assert worst <= lim_row, f"{what}: worst row relative L2 error {worst} > {lim_row}"
    if lse is not None:
        lse = np.asarray(lse, np.float64)
        lse_ref = np.asarray(lse_ref, np.float64)
        both_inf = np.isneginf(lse) & np.isneginf(lse_ref)
        d = np.abs(np.where(both_inf, 0.0, lse) - np.where(both_inf, 0.0, lse_ref))
        ml = float(d.max()) if d.size else 0.0
        note(f"  {what}: lse max_abs={ml:.3e}")
        assert ml <= (1e-5 if f32 else LSE_MAX_ABS), f"{what}: LSE error {ml}"


def mla_device_inputs(x, w, torch):
    """Device tensors for an 'mla' workload from li.generate()."""
    kv = to_dev(x["kv"], torch)
    width = w.n_lat * w.d_c + w.d_rope
    flat = kv.reshape(-1)
    return dict(q_nope=to_dev(x["q_nope"], torch), q_rope=to_dev(x["q_rope"], torch),
                c_kv=flat, k_rope=flat[w.n_lat * w.d_c:], kv_tok_stride=width,
                rope_tok_stride=width,
                block_table=torch.from_numpy(x["block_table"]).cuda(),
                seqlens=torch.from_numpy(x["seqlens"]).cuda(), kv=kv)


def run_mla(lkv, w, d, x=None, **kw):
    return lkv.lkv_mla_decode(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["block_table"],
                              d["seqlens"], n_latent=w.n_lat, page_size=w.page_size,
                              softmax_scale=w.scale, causal=w.causal,
                              kv_tok_stride=d["kv_tok_stride"],
                              rope_tok_stride=d["rope_tok_stride"],
                              seqlens_host=None if x is None else x["seqlens"], **kw)


def oracle_mla(oracle, w, x, rows=None, q_nope=None):
    width = w.n_lat * w.d_c + w.d_rope
    kv = x["kv"].reshape(-1)
    return oracle.mla_decode(x["q_nope"] if q_nope is None else q_nope, x["q_rope"], kv,
                             kv[w.n_lat * w.d_c:], x["block_table"], x["seqlens"],
                             n_lat=w.n_lat, d_c=w.d_c, d_rope=w.d_rope, page_size=w.page_size,
                             scale=w.scale, causal=w.causal, kv_tok_stride=width,
                             rope_tok_stride=width, rows=rows)


def small_mla(seed, *, B=3, h_q=128, s_q=1, n_lat=1, d_c=512, d_rope=64, page=64, seqlens=None,
              table="fragmented", causal=True, dtype="bf16", max_pages=None, cache=""):
    rng = np.random.default_rng(seed)
    if seqlens is None:
        seqlens = rng.integers(s_q, 700, size=B)
    w = li.Workload(name=f"small{seed}", kind="mla", dtype=dtype, B=len(seqlens), h_q=h_q, s_q=s_q,
                    page_size=page, n_lat=n_lat, d_c=d_c, d_rope=d_rope,
                    seqlens=tuple(int(v) for v in seqlens), table=table, causal=causal,
                    max_pages=max_pages, scale=1 / math.sqrt(d_c + d_rope), seed=seed,
                    cache=cache)
    return w, li.generate(w)


def dequantised(oracle, x, cache_keys, q_keys):
    """Copy of generate()'s output for the oracle when the caches hold E4M3
    codes: caches as float32 values through the oracle's decoding of all 256
    codes (exact: the scale is a power of two), bf16 queries widened to
    float32 so that every oracle input shares one dtype."""
    lut = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8), x["kv_scale"]).astype(np.float32)
    y = dict(x)
    for k in cache_keys:
        y[k] = lut[x[k]]
    for k in q_keys:
        y[k] = li.bf16_bits_to_f32(x[k])
    return y


def rows_of(out, rows):
    B, s_q, h_q = out.shape[:3]
    return out.reshape(B * s_q * h_q, *out.shape[3:])[rows]
