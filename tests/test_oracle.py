"""Pins for the fp64 oracle: each check ties the oracle to something other
than itself.

  * a library attention routine (torch scaled_dot_product_attention, fp64,
    CPU) on caches gathered contiguous through the block table;
  * closed forms (zero query -> mean of the visible latents, LSE = ln n;
    one visible token -> that token);
  * the pages' algebraic claims: absorbed == explicit (GQLA technical
    summary section 2 and the X post's absorb trick), GQLA absorbed ==
    grouped on the same weights (GQLA section 2: two algebraically
    equivalent paths), "mixing can learn copying" (X post) with selection
    up-projections;
  * split-KV invariance (any split plan, empty splits included);
  * physical-page permutation invariance of the block-table gather.
"""
import math

import numpy as np
import pytest
import torch

import lkv_inputs as li

torch.set_default_dtype(torch.float64)


def _f64(a):
    if a.dtype == np.uint16:
        return li.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _tiny(seed, B=3, h_q=8, s_q=1, n_lat=1, d_c=32, d_rope=8, page=16, dtype="f32",
          seqlens=None, table="shuffled"):
    rng = np.random.default_rng(seed)
    if seqlens is None:
        seqlens = rng.integers(max(1, s_q), 71, size=B)
    w = li.Workload(name="t", kind="mla", dtype=dtype, B=B, h_q=h_q, s_q=s_q, page_size=page,
                    n_lat=n_lat, d_c=d_c, d_rope=d_rope, seqlens=tuple(int(x) for x in seqlens),
                    table=table, scale=1 / math.sqrt(d_c + d_rope), seed=seed)
    return w, li.generate(w)


def _gather(cache, table, b, n, page):
    """Contiguous copy of the first n tokens of sequence b (independent of the
    oracle's own gather)."""
    idx = [(table[b, j // page], j % page) for j in range(n)]
    return np.stack([cache[p, s] for p, s in idx]) if n else cache[:0, 0]


def _sdpa_rows(q, k, v, scale, visible):
    """Library attention for one (b, latent) block: q [R, D], k [n, D],
    v [n, Dv]; visible[r] = number of cache tokens row r sees."""
    n = k.shape[0]
    mask = torch.arange(n)[None, :] < torch.as_tensor(visible)[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(q)[None], torch.as_tensor(k)[None], torch.as_tensor(v)[None],
        attn_mask=mask[None], scale=scale)[0]
    s = (torch.as_tensor(q) @ torch.as_tensor(k).T) * scale
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    return o.numpy(), lse.numpy()


def _mla_via_sdpa(w, x, causal=True):
    P, dc, nl = w.page_size, w.d_c, w.n_lat
    kv = _f64(x["kv"])
    qn, qr = _f64(x["q_nope"]), _f64(x["q_rope"])
    B, s_q, h_q = w.B, w.s_q, w.h_q
    hpl = h_q // nl
    out = np.zeros((B, s_q, h_q, dc))
    lse = np.zeros((B, s_q, h_q))
    for b in range(B):
        L = int(x["seqlens"][b])
        g = _gather(kv, x["block_table"], b, L, P)
        for l in range(nl):
            c = g[:, l * dc:(l + 1) * dc]
            r = g[:, nl * dc:]
            k = np.concatenate([c, r], axis=1)
            heads = slice(l * hpl, (l + 1) * hpl)
            q = np.concatenate([qn[b, :, heads], qr[b, :, heads]], axis=-1).reshape(s_q * hpl, -1)
            vis = np.repeat([L - s_q + t + 1 if causal else L for t in range(s_q)], hpl)
            o, ls = _sdpa_rows(q, k, c, w.scale, vis)
            out[b, :, heads] = o.reshape(s_q, hpl, dc)
            lse[b, :, heads] = ls.reshape(s_q, hpl)
    return out, lse


def _oracle_mla(oracle_lib, w, x, causal=True, **kw):
    nl, dc = w.n_lat, w.d_c
    kv = x["kv"]
    return oracle_lib.mla_decode(x["q_nope"], x["q_rope"], kv[..., :nl * dc].copy(),
                                 kv[..., nl * dc:].copy(), x["block_table"], x["seqlens"],
                                 n_lat=nl, d_c=dc, d_rope=w.d_rope, page_size=w.page_size,
                                 scale=w.scale, causal=causal, **kw)


# ---------------------------------------------------------------- O1 vs SDPA
@pytest.mark.parametrize("seed,s_q,n_lat,dtype,causal", [
    (10, 1, 1, "f32", True), (11, 2, 1, "f32", True), (12, 2, 1, "bf16", False),
    (13, 1, 2, "bf16", True), (14, 3, 2, "f32", True), (15, 2, 1, "f32", False)])
def test_mla_matches_library_attention(oracle_lib, seed, s_q, n_lat, dtype, causal):
    w, x = _tiny(seed, s_q=s_q, n_lat=n_lat, dtype=dtype)
    o, l = _oracle_mla(oracle_lib, w, x, causal)
    o2, l2 = _mla_via_sdpa(w, x, causal)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, l2, rtol=1e-12, atol=1e-12)


def test_mla_packed_cache_strides(oracle_lib):
    """The packed [.., n_lat*d_c + d_rope] cache read through strides gives the
    same result as separate contiguous arrays."""
    w, x = _tiny(20, s_q=2, n_lat=2)
    nl, dc = w.n_lat, w.d_c
    width = nl * dc + w.d_rope
    kv = x["kv"]
    o1, l1 = oracle_lib.mla_decode(x["q_nope"], x["q_rope"], kv, kv.reshape(-1)[nl * dc:],
                                   x["block_table"], x["seqlens"], n_lat=nl, d_c=dc,
                                   d_rope=w.d_rope, page_size=w.page_size, scale=w.scale,
                                   kv_tok_stride=width, rope_tok_stride=width)
    o2, l2 = _oracle_mla(oracle_lib, w, x)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------- closed forms
def test_zero_query_gives_mean_and_ln_n(oracle_lib):
    w, x = _tiny(30, s_q=2, n_lat=2)
    x["q_nope"][:] = 0
    x["q_rope"][:] = 0
    o, l = _oracle_mla(oracle_lib, w, x)
    kv = _f64(x["kv"])
    hpl = w.h_q // w.n_lat
    for b in range(w.B):
        L = int(x["seqlens"][b])
        g = _gather(kv, x["block_table"], b, L, w.page_size)
        for t in range(w.s_q):
            n = L - w.s_q + t + 1
            for h in range(w.h_q):
                lat = h // hpl
                mean = g[:n, lat * w.d_c:(lat + 1) * w.d_c].mean(axis=0)
                np.testing.assert_allclose(o[b, t, h], mean, rtol=1e-12, atol=1e-13)
                assert abs(l[b, t, h] - math.log(n)) < 1e-12


def test_single_visible_token(oracle_lib):
    w, x = _tiny(31, B=2, s_q=1, seqlens=[1, 1])
    o, l = _oracle_mla(oracle_lib, w, x)
    kv = _f64(x["kv"])
    for b in range(2):
        p = x["block_table"][b, 0]
        c0 = kv[p, 0, :w.d_c]
        r0 = kv[p, 0, w.d_c:]
        qn, qr = _f64(x["q_nope"])[b, 0], _f64(x["q_rope"])[b, 0]
        for h in range(w.h_q):
            np.testing.assert_array_equal(o[b, 0, h], c0)
            expect = w.scale * (float(qn[h] @ c0) + float(qr[h] @ r0))
            assert abs(l[b, 0, h] - expect) < 1e-12 * max(1.0, abs(expect))


def test_softmax_weights_sum_to_one(oracle_lib):
    w, x = _tiny(32, s_q=2, n_lat=1)
    kv = x["kv"]
    for b in range(w.B):
        for t in range(w.s_q):
            for h in (0, w.h_q - 1):
                p = oracle_lib.mla_row_weights(x["q_nope"], x["q_rope"], kv[..., :w.d_c].copy(),
                                               kv[..., w.d_c:].copy(), x["block_table"],
                                               x["seqlens"], b, t, h, n_lat=1, d_c=w.d_c,
                                               d_rope=w.d_rope, page_size=w.page_size,
                                               scale=w.scale)
                assert p.size == int(x["seqlens"][b]) - w.s_q + t + 1
                assert abs(p.sum() - 1.0) < 1e-12
                assert (p >= 0).all()


def test_empty_row_gives_zero_and_neg_inf(oracle_lib):
    w, x = _tiny(33, B=2, s_q=1, seqlens=[5, 9])
    x["seqlens"][0] = 0
    o, l = _oracle_mla(oracle_lib, w, x)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    assert np.isfinite(o[1]).all()


# ------------------------------------------------------ page permutation
def test_physical_page_permutation_is_exact(oracle_lib):
    w, x = _tiny(40, s_q=2)
    o1, l1 = _oracle_mla(oracle_lib, w, x)
    rng = np.random.default_rng(0)
    perm = rng.permutation(x["num_pages"])          # new page i holds old page perm[i]
    inv = np.argsort(perm)
    y = dict(x)
    y["kv"] = x["kv"][perm]
    bt = x["block_table"].copy()
    bt[bt >= 0] = inv[bt[bt >= 0]]
    y["block_table"] = bt
    o2, l2 = _oracle_mla(oracle_lib, w, y)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ---------------------------------------------------------------- split-KV
@pytest.mark.parametrize("plan", ["halves", "sevenths", "with_empty", "single"])
def test_split_combine_equals_single_pass(oracle_lib, plan):
    w, x = _tiny(50, B=3, s_q=2, n_lat=2, seqlens=[70, 17, 33])
    full_o, full_l = _oracle_mla(oracle_lib, w, x)
    Lmax = int(x["seqlens"].max())
    if plan == "halves":
        cuts = [0, Lmax // 2, Lmax]
    elif plan == "sevenths":
        cuts = sorted(set([0] + [Lmax * k // 7 for k in range(1, 7)] + [Lmax]))
    elif plan == "with_empty":
        cuts = [0, 0, 5, 5, 40, Lmax + 10, Lmax + 20]
    else:
        cuts = [0, Lmax]
    parts_o, parts_l, offs = [], [], [0]
    for b in range(w.B):
        for k in range(len(cuts) - 1):
            lo = np.full(w.B, cuts[k], np.int32)
            hi = np.full(w.B, cuts[k + 1], np.int32)
            o, l = _oracle_mla(oracle_lib, w, x, range_lo=lo, range_hi=hi)
            parts_o.append(o[b])
            parts_l.append(l[b])
        offs.append(len(parts_o))
    co, cl = oracle_lib.lse_combine(np.stack(parts_o), np.stack(parts_l), np.array(offs))
    np.testing.assert_allclose(co, full_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(cl, full_l, rtol=1e-12, atol=1e-13)


def test_combine_all_empty_gives_zero(oracle_lib):
    o = np.random.default_rng(1).standard_normal((2, 1, 2, 4))
    l = np.full((2, 1, 2), -np.inf)
    co, cl = oracle_lib.lse_combine(o, l, np.array([0, 2]))
    assert np.all(co == 0) and np.all(np.isneginf(cl))


# ---------------------------------------------------------------- GQA (O3)
def _gqa_inputs(seed, B=2, h_q=8, n_kv=2, d_h=16, d_rope=8, s_q=2, page=16, dtype="f32"):
    rng = np.random.default_rng(seed)
    w = li.Workload(name="g", kind="gqa", dtype=dtype, B=B, h_q=h_q, s_q=s_q, page_size=page,
                    n_kv=n_kv, d_h=d_h, d_rope=d_rope,
                    seqlens=tuple(int(v) for v in rng.integers(s_q, 60, size=B)),
                    scale=1 / math.sqrt(d_h + d_rope), seed=seed)
    return w, li.generate(w)


@pytest.mark.parametrize("n_kv,d_rope,s_q", [(2, 8, 2), (1, 0, 1), (8, 0, 1), (4, 8, 3)])
def test_gqa_matches_library_attention(oracle_lib, n_kv, d_rope, s_q):
    w, x = _gqa_inputs(60 + n_kv, n_kv=n_kv, d_rope=d_rope, s_q=s_q)
    o, l = oracle_lib.gqa_decode(x["q"], x["k_cache"], x["v_cache"], x["block_table"],
                                 x["seqlens"], n_kv=n_kv, d_h=w.d_h, page_size=w.page_size,
                                 scale=w.scale, q_rope=x.get("q_rope"), k_rope=x.get("k_rope"),
                                 d_rope=d_rope)
    K, V = _f64(x["k_cache"]), _f64(x["v_cache"])
    R = _f64(x["k_rope"]) if d_rope else None
    q = _f64(x["q"])
    qr = _f64(x["q_rope"]) if d_rope else None
    hpg = w.h_q // n_kv
    for b in range(w.B):
        L = int(x["seqlens"][b])
        kb = _gather(K, x["block_table"], b, L, w.page_size)
        vb = _gather(V, x["block_table"], b, L, w.page_size)
        rb = _gather(R, x["block_table"], b, L, w.page_size) if d_rope else None
        for h in range(w.h_q):
            g = h // hpg
            k = np.concatenate([kb[:, g], rb], axis=1) if d_rope else kb[:, g]
            qq = np.concatenate([q[b, :, h], qr[b, :, h]], axis=-1) if d_rope else q[b, :, h]
            vis = [L - s_q + t + 1 for t in range(s_q)]
            oo, ll = _sdpa_rows(qq, k, vb[:, g], w.scale, vis)
            np.testing.assert_allclose(o[b, :, h], oo, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(l[b, :, h], ll, rtol=1e-12, atol=1e-12)


# ------------------------------------------------- absorb / explicit / GQLA
def _latent_case(seed, B=2, h_q=8, n_w=8, d_c=32, d_h=8, d_rope=8, s_q=2, page=16):
    rng = np.random.default_rng(seed)
    w, x = _tiny(seed, B=B, h_q=h_q, s_q=s_q, d_c=d_c, d_rope=d_rope, page=page, dtype="f32")
    kv = x["kv"].astype(np.float64)
    q_h = rng.standard_normal((B, s_q, h_q, d_h))
    qr = rng.standard_normal((B, s_q, h_q, d_rope))
    wuk = rng.standard_normal((n_w, d_c, d_h)) / math.sqrt(d_c)
    wuv = rng.standard_normal((n_w, d_c, d_h)) / math.sqrt(d_c)
    return w, x, kv, q_h, qr, wuk, wuv


def test_absorb_and_up_project_match_matmul(oracle_lib):
    _, _, _, q_h, _, wuk, wuv = _latent_case(70, n_w=4)
    qa = oracle_lib.absorb_query(q_h, wuk)
    hpw = q_h.shape[2] // 4
    for h in range(q_h.shape[2]):
        np.testing.assert_allclose(qa[:, :, h], q_h[:, :, h] @ wuk[h // hpw].T, rtol=1e-13,
                                   atol=1e-13)
    o_lat = np.random.default_rng(1).standard_normal(qa.shape)
    up = oracle_lib.up_project(o_lat, wuv)
    for h in range(q_h.shape[2]):
        np.testing.assert_allclose(up[:, :, h], o_lat[:, :, h] @ wuv[h // hpw], rtol=1e-13,
                                   atol=1e-13)


@pytest.mark.parametrize("n_w", [8, 2])
def test_absorbed_equals_explicit(oracle_lib, n_w):
    """GQLA section 2 / X post: folding W_UK into q and W_UV into the output
    leaves the attention unchanged (n_w = h_q: MLA; n_w = g: GQLA)."""
    w, x, kv, q_h, qr, wuk, wuv = _latent_case(71, n_w=n_w)
    d_c = w.d_c
    qa = oracle_lib.absorb_query(q_h, wuk)
    o_lat, l_abs = oracle_lib.mla_decode(qa, qr, kv[..., :d_c].copy(), kv[..., d_c:].copy(),
                                         x["block_table"], x["seqlens"], n_lat=1, d_c=d_c,
                                         d_rope=w.d_rope, page_size=w.page_size, scale=w.scale)
    o_abs = oracle_lib.up_project(o_lat, wuv)
    o_exp, l_exp = oracle_lib.mla_explicit(q_h, qr, wuk, wuv, kv[..., :d_c].copy(),
                                           kv[..., d_c:].copy(), x["block_table"], x["seqlens"],
                                           page_size=w.page_size, scale=w.scale)
    np.testing.assert_allclose(o_abs, o_exp, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(l_abs, l_exp, rtol=1e-10, atol=1e-11)


def test_gqla_absorbed_equals_grouped(oracle_lib):
    """GQLA section 2: the MQA-absorbed path and the GQA path (latent
    expanded once into g groups, shared RoPE key) agree on the same weights."""
    g = 2
    w, x, kv, q_h, qr, wuk, wuv = _latent_case(72, n_w=g)
    d_c, d_h = w.d_c, q_h.shape[-1]
    qa = oracle_lib.absorb_query(q_h, wuk)
    o_lat, l_abs = oracle_lib.mla_decode(qa, qr, kv[..., :d_c].copy(), kv[..., d_c:].copy(),
                                         x["block_table"], x["seqlens"], n_lat=1, d_c=d_c,
                                         d_rope=w.d_rope, page_size=w.page_size, scale=w.scale)
    o_abs = oracle_lib.up_project(o_lat, wuv)
    K, V = oracle_lib.expand_latent(kv[..., :d_c].copy(), wuk, wuv, x["block_table"],
                                    x["seqlens"], page_size=w.page_size,
                                    num_pages=x["num_pages"])
    K = np.nan_to_num(K)
    V = np.nan_to_num(V)
    o_grp, l_grp = oracle_lib.gqa_decode(q_h, K, V, x["block_table"], x["seqlens"], n_kv=g,
                                         d_h=d_h, page_size=w.page_size, scale=w.scale,
                                         q_rope=qr, k_rope=kv[..., d_c:].copy(), d_rope=w.d_rope)
    np.testing.assert_allclose(o_abs, o_grp, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(l_abs, l_grp, rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("g", [1, 2, 8])
def test_mixing_learns_copying(oracle_lib, g):
    """X post: 'mixing' can learn 'copying'.  With d_c = g*d_h and W_UK[k] =
    W_UV[k] = the selection of latent slice k, MLA equals GQA whose K and V of
    group k are that slice (g = 1: MQA; g = h_q: MHA)."""
    h_q, d_h = 8, 8
    d_c = g * d_h
    w, x = _tiny(80 + g, B=2, h_q=h_q, s_q=2, d_c=d_c, d_rope=8, dtype="f32")
    kv = x["kv"].astype(np.float64)
    sel = np.zeros((g, d_c, d_h))
    for k in range(g):
        sel[k, k * d_h:(k + 1) * d_h, :] = np.eye(d_h)
    rng = np.random.default_rng(g)
    q_h = rng.standard_normal((2, 2, h_q, d_h))
    qr = rng.standard_normal((2, 2, h_q, 8))
    qa = oracle_lib.absorb_query(q_h, sel)
    o_lat, l1 = oracle_lib.mla_decode(qa, qr, kv[..., :d_c].copy(), kv[..., d_c:].copy(),
                                      x["block_table"], x["seqlens"], n_lat=1, d_c=d_c, d_rope=8,
                                      page_size=w.page_size, scale=w.scale)
    o1 = oracle_lib.up_project(o_lat, sel)
    c = np.ascontiguousarray(kv[..., :d_c]).reshape(kv.shape[0], kv.shape[1], g, d_h)
    o2, l2 = oracle_lib.gqa_decode(q_h, c, c, x["block_table"], x["seqlens"], n_kv=g, d_h=d_h,
                                   page_size=w.page_size, scale=w.scale, q_rope=qr,
                                   k_rope=kv[..., d_c:].copy(), d_rope=8)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-13)


def test_expand_matches_matmul(oracle_lib):
    w, x, kv, _, _, wuk, wuv = _latent_case(90, n_w=3)
    d_c = w.d_c
    K, V = oracle_lib.expand_latent(x["kv"][..., :d_c].copy(), wuk, wuv, x["block_table"],
                                    x["seqlens"], page_size=w.page_size,
                                    num_pages=x["num_pages"], kv_tok_stride=None)
    for b in range(w.B):
        L = int(x["seqlens"][b])
        for j in range(L):
            p, s = x["block_table"][b, j // w.page_size], j % w.page_size
            c = kv[p, s, :d_c]
            for k in range(3):
                np.testing.assert_allclose(K[p, s, k], c @ wuk[k], rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(V[p, s, k], c @ wuv[k], rtol=1e-12, atol=1e-12)
    valid = li.valid_slot_mask(x["block_table"], x["seqlens"], w.page_size, x["num_pages"])
    assert np.isnan(K[~valid]).all() and np.isfinite(K[valid]).all()


def test_expand_start_pos_skips_prefix(oracle_lib):
    w, x, kv, _, _, wuk, wuv = _latent_case(91, n_w=2)
    sp = np.array([3, 0], np.int32)
    K, _ = oracle_lib.expand_latent(x["kv"][..., :w.d_c].copy(), wuk, wuv, x["block_table"],
                                    x["seqlens"], page_size=w.page_size,
                                    num_pages=x["num_pages"], start_pos=sp)
    for j in range(3):
        p, s = x["block_table"][0, j // w.page_size], j % w.page_size
        assert np.isnan(K[p, s]).all()
    p, s = x["block_table"][0, 3 // w.page_size], 3 % w.page_size
    assert np.isfinite(K[p, s]).all()


def test_tiny_fp32_workload_runs_fast(oracle_lib):
    """The tiny fp32 workload (B=2, h_q=16, d_c=64, d_rope=16, L={200,256},
    page 16) finishes in well under a second and is NaN-free despite poisoned
    tails."""
    import time
    w = li.workload("tiny_mla_fp32")
    x = li.generate(w)
    t0 = time.perf_counter()
    o, l = _oracle_mla(oracle_lib, w, x)
    assert time.perf_counter() - t0 < 1.0
    assert np.isfinite(o).all() and np.isfinite(l).all()
    assert x["num_pages"] == 29


def test_append_tokens_rebuilds_the_generated_cache(oracle_lib):
    """Appending every valid token of a generated batch, a few tokens per
    step from an empty cache, reproduces the paged layout that lkv_inputs
    builds on its own (its valid slots bit for bit; the other slots stay
    untouched)."""
    w = li.Workload(name="app", kind="mla", dtype="bf16", B=3, h_q=16, s_q=1, page_size=16,
                    n_lat=1, d_c=64, d_rope=16, seqlens=(37, 16, 5), table="fragmented",
                    scale=0.1, seed=31)
    x = li.generate(w)
    kv = x["kv"]  # [num_pages, page_size, width], unused slots NaN
    npg, P, width = kv.shape
    bt, sl = x["block_table"], x["seqlens"]
    # the logical rows of each sequence, read through the table
    logical = [np.stack([kv[bt[b, j // P], j % P] for j in range(int(sl[b]))]) for b in range(w.B)]
    sentinel = np.uint16(0x1234)
    cache = np.full(npg * P * width, sentinel, np.uint16)
    step = 3
    for L_done in range(0, int(sl.max()), step):
        s_q = step
        lens = np.minimum(sl, L_done + s_q).astype(np.int32)
        src = np.full((w.B, s_q, width), sentinel, np.uint16)
        for b in range(w.B):
            for t in range(s_q):
                j = int(lens[b]) - s_q + t
                if j >= L_done:  # a new token of this step
                    src[b, t] = logical[b][j]
                elif j >= 0:     # already written: write the same row again
                    src[b, t] = logical[b][j]
        cache = oracle_lib.append_tokens(src, cache, bt, lens, page_size=P, tok_stride=width)
    got = cache.reshape(npg, P, width)
    valid = li.valid_slot_mask(bt, sl, P, npg)
    assert np.array_equal(got[valid], kv[valid])
    assert (got[~valid] == sentinel).all()


def test_e4m3_decode_matches_the_format_definition(oracle_lib):
    """OCP E4M3 values fixed by the format: 1.0, the largest normal 448, the
    smallest normal 2^-6, the smallest subnormal 2^-9, the largest subnormal
    7 * 2^-9, signed zero, NaN; and the input generator's encoder is the
    inverse of the decoder on every finite code."""
    f = oracle_lib.e4m3_to_f64
    fixed = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x00: 0.0, 0xB8: -1.0, 0xFE: -448.0, 0x40: 2.0, 0x3C: 1.5}
    for code, val in fixed.items():
        assert f(np.array([code]))[0] == val, hex(code)
    assert np.isnan(f(np.array([0x7F, 0xFF]))).all()
    assert np.signbit(f(np.array([0x80]))[0])
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(li.to_e4m3_bits(f(codes)), codes)
    # rounding: halfway between 1.0 (0x38) and 1.125 (0x39) goes to the even code
    assert li.to_e4m3_bits(np.array([1.0625]))[0] == 0x38
    assert li.to_e4m3_bits(np.array([1.1875]))[0] == 0x3A
    assert li.to_e4m3_bits(np.array([1000.0]))[0] == 0x7E


def test_e4m3_encode_is_nearest_code(oracle_lib):
    """The oracle's E4M3 encoding: every finite code round-trips through its
    value; every midpoint between adjacent codes goes to the even code and
    points just off it to the nearer one; magnitudes past 448 saturate;
    signed zero and NaN follow the format."""
    enc, dec = oracle_lib.e4m3_from_f64, oracle_lib.e4m3_to_f64
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(enc(dec(finite)), finite)
    pos = np.arange(0x7F, dtype=np.uint8)
    v = dec(pos)
    mid = (v[:-1] + v[1:]) / 2
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(enc(mid), even)
    step = v[1:] - v[:-1]
    assert np.array_equal(enc(mid - step / 8), pos[:-1])
    assert np.array_equal(enc(mid + step / 8), pos[1:])
    assert np.array_equal(enc(-mid), even | 0x80)
    assert enc(np.array([448.0]))[0] == 0x7E and enc(np.array([1e6]))[0] == 0x7E
    assert enc(np.array([-470.0]))[0] == 0xFE
    assert enc(np.array([-0.0]))[0] == 0x80 and enc(np.array([0.0]))[0] == 0x00
    assert enc(np.array([2.0 ** -10]))[0] == 0x00            # tie between 0 and 2^-9
    assert enc(np.array([3 * 2.0 ** -10]))[0] == 0x02        # tie between 2^-9 and 2^-8
    assert (enc(np.array([np.nan]))[0] & 0x7F) == 0x7F
