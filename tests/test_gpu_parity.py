"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
the same seeded inputs.

Small cases span several 64-token tiles, ragged tails, NaN-poisoned unused
slots and pages, both s_q readings (causal and not), several split plans and
every compiled head width.  Full-size cases run the workloads at their real
shapes in the launch configuration the benchmark times and compare sampled
rows with the oracle computed row by row.
"""
import math

import numpy as np
import pytest

import lkv_inputs as li
from tests.gpu_common import (assert_close, dequantised, from_dev, mla_device_inputs, note,
                              oracle_mla, rows_of, run_mla, small_mla, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import latent_kv_decode_amd as m
    m.load_library()
    return m


@pytest.fixture(scope="module")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


# ------------------------------------------------------------------ fp32 tiny
def test_tiny_fp32_workload(lkv, oracle):
    w = li.workload("tiny_mla_fp32")
    x = li.generate(w)
    note("case tiny_mla_fp32")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d)
    torch.cuda.synchronize()
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, f32=True, what="tiny fp32")


@pytest.mark.parametrize("s_q,causal,n_lat", [(1, True, 1), (2, True, 2), (3, False, 1)])
def test_fp32_variants(lkv, oracle, s_q, causal, n_lat):
    w, x = small_mla(100 + s_q, B=3, h_q=16, s_q=s_q, n_lat=n_lat, d_c=64, d_rope=16, page=16,
                     causal=causal, dtype="f32")
    note(f"case fp32 s_q={s_q} causal={causal} n_lat={n_lat}")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d)
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, f32=True, what="fp32")


@pytest.mark.parametrize("d_c,d_rope", [(64, 6), (62, 16), (30, 4)])
def test_fp32_rows_not_16_byte_chunks(lkv, oracle, d_c, d_rope):
    """Token rows whose segments are not whole 16-byte chunks (a RoPE width
    of 6, a latent width of 62 or 30 floats): the float32 kernel stages them
    with 4-byte loads instead of 16-byte ones."""
    w, x = small_mla(150 + d_c + d_rope, B=3, h_q=16, s_q=1, d_c=d_c, d_rope=d_rope, page=16,
                     seqlens=[1, 130, 257], dtype="f32")
    note(f"case fp32 rows d_c={d_c} d_rope={d_rope}")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d)
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, f32=True, what="fp32 rows")


# ------------------------------------------------------------------ bf16 MLA
@pytest.mark.parametrize("s_q,causal,splits", [
    (1, True, 0), (1, True, 1), (1, True, 2), (1, True, 7), (1, True, 1000),
    (2, True, 0), (2, True, 5), (2, False, 3), (3, True, 0)])
def test_mla_small(lkv, oracle, s_q, causal, splits):
    w, x = small_mla(200 + 10 * s_q + splits % 97, B=4, s_q=s_q, causal=causal,
                     seqlens=[1 + (s_q - 1), 63, 65, 700] if s_q < 3 else [3, 64, 129, 400])
    note(f"case mla_small s_q={s_q} causal={causal} splits={splits} seqlens={list(x['seqlens'])}")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d, x=x if splits % 2 == 0 else None, num_splits=splits)
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"mla s_q={s_q} splits={splits}")


def test_mla_split_plans_agree(lkv, oracle):
    """Forced share counts {1, 2, 7, many} all meet the oracle and agree with
    each other closely."""
    w, x = small_mla(250, B=3, s_q=2, seqlens=[900, 31, 444])
    d = mla_device_inputs(x, w, torch)
    ro, rl = oracle_mla(oracle, w, x)
    outs = []
    for splits in (1, 2, 7, 64):
        note(f"case split plan {splits}")
        out, lse = run_mla(lkv, w, d, num_splits=splits)
        assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"splits={splits}")
        outs.append(from_dev(out))
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 2e-2


def _shares(seqlens, splits):
    """Shares each sequence is cut into when the concatenated 64-token tiles
    of the batch (an empty sequence counts one tile) are cut into `splits`
    equal shares."""
    tiles = [max(1, -(-int(L) // 64)) for L in seqlens]
    chunk = -(-sum(tiles) // splits)
    out, cu = [], 0
    for nb in tiles:
        out.append((cu + nb - 1) // chunk - cu // chunk + 1)
        cu += nb
    return out


def test_mla_split_share_counts(lkv, oracle):
    """128 query rows per latent head, with plans that cut the sequences into
    1, 2, 3, 4 and more shares (an empty sequence among them).  Every plan
    runs with and without host lengths (with them the combine pass is skipped
    when no sequence is cut), twice in a row on the same workspace, into
    outputs poisoned with NaN so that a row left unwritten fails."""
    seqlens = [2000, 130, 700, 64, 5, 1500, 300, 1, 2600, 190]
    w, x = small_mla(260, B=len(seqlens), seqlens=seqlens)
    x["seqlens"][4] = 0
    d = mla_device_inputs(x, w, torch)
    ro, rl = oracle_mla(oracle, w, x)
    seen = set()
    for splits in (5, 9, 16, 23, 64):
        shares = _shares(x["seqlens"], splits)
        seen.update(shares)
        for host in (True, False):
            for rep in range(2):
                note(f"case share counts splits={splits} shares={shares} host={host} rep={rep}")
                out = torch.full((w.B, 1, w.h_q, w.d_c), float("nan"), dtype=torch.bfloat16,
                                 device="cuda")
                lse = torch.full((w.B, 1, w.h_q), float("nan"), dtype=torch.float32, device="cuda")
                out, lse = run_mla(lkv, w, d, x=x if host else None, num_splits=splits, out=out,
                                   lse=lse)
                assert_close(from_dev(out), ro, from_dev(lse), rl,
                             what=f"splits={splits} host={host} rep={rep}")
    assert {1, 2, 3, 4} <= seen and max(seen) > 4, seen


@pytest.mark.parametrize("h_q,n_lat,d_c,s_q,causal", [
    (32, 2, 256, 1, True), (16, 1, 512, 1, True), (64, 1, 128, 1, True), (48, 1, 512, 1, True),
    (32, 8, 128, 1, True),
    # several query tokens with and without causal masking among them on the
    # row-tiled kernel (at most 32 rows per latent head)
    (32, 2, 256, 2, False), (16, 1, 512, 2, False), (32, 8, 128, 4, False),
    (16, 1, 512, 2, True), (32, 8, 128, 4, True)])
def test_mla_head_shapes(lkv, oracle, h_q, n_lat, d_c, s_q, causal):
    """GLA-2 (two latent heads, shared RoPE key), few heads (one 16-row tile),
    a narrow latent, a head count that leaves a padded row tile, and GTA
    (eight tied key/value groups of 128 as latent heads, shared RoPE key);
    the row-tiled kernel with s_q > 1, causal and not."""
    w, x = small_mla(300 + h_q + 7 * s_q + (0 if causal else 3), B=3, h_q=h_q, n_lat=n_lat,
                     d_c=d_c, s_q=s_q, causal=causal, seqlens=[s_q + 76, 300, 129])
    note(f"case mla_heads h_q={h_q} n_lat={n_lat} d_c={d_c} s_q={s_q} causal={causal}")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d, x=x)
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl,
                 what=f"mla h_q={h_q} n_lat={n_lat} s_q={s_q} causal={causal}")


@pytest.mark.parametrize("h_q,d_c,d_rope,s_q,splits", [
    (64, 256, 64, 1, 0), (128, 512, 0, 1, 0), (64, 256, 0, 2, 3), (128, 512, 64, 2, 0),
    (96, 512, 64, 1, 5), (128, 512, 64, 4, 0)])
def test_mla_many_rows_widths(lkv, oracle, h_q, d_c, d_rope, s_q, splits):
    """Latent and RoPE widths (512/256, with and without RoPE) with many query
    rows per latent head, including a row count that is not a multiple of
    the rows one work-group takes."""
    w, x = small_mla(500 + h_q + d_c + d_rope + s_q, B=3, h_q=h_q, d_c=d_c, d_rope=d_rope, s_q=s_q,
                     seqlens=[s_q + 60, 257, 640])
    note(f"case mla_many_rows h_q={h_q} d_c={d_c} d_rope={d_rope} s_q={s_q} splits={splits}")
    d = mla_device_inputs(x, w, torch)
    out, lse = lkv.lkv_mla_decode(d["q_nope"], d["q_rope"] if d_rope else None, d["c_kv"],
                                  d["k_rope"] if d_rope else None, d["block_table"], d["seqlens"],
                                  page_size=w.page_size, softmax_scale=w.scale, causal=w.causal,
                                  kv_tok_stride=d["kv_tok_stride"],
                                  rope_tok_stride=d["rope_tok_stride"] if d_rope else None,
                                  num_splits=splits)
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"mla h_q={h_q} d_c={d_c} d_rope={d_rope}")


@pytest.mark.parametrize("page", [16, 32, 128, 48])
def test_mla_page_sizes(lkv, oracle, page):
    w, x = small_mla(400 + page, B=3, page=page, seqlens=[100, 257, 31])
    note(f"case page_size={page}")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d, x=x)
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"page={page}")


def test_mla_empty_and_short_rows(lkv, oracle):
    """L_b = 0 (no visible token), L_b < s_q under causal masking (row t=0
    sees nothing), and L_b = 1: O = 0 / LSE = -inf where nothing is seen."""
    w, x = small_mla(450, B=4, s_q=2, seqlens=[2, 5, 9, 70])
    x["seqlens"] = np.array([0, 1, 9, 70], np.int32)
    note("case empty/short rows")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d, x=x)
    ro, rl = oracle_mla(oracle, w, x)
    o, l = from_dev(out), from_dev(lse)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    assert np.all(o[1, 0] == 0) and np.all(np.isneginf(l[1, 0]))
    assert_close(o, ro, l, rl, what="empty/short")


def test_batch_zero_is_noop(lkv):
    q = torch.zeros((0, 1, 128, 512), dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros((0, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((64, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    sl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out, lse = lkv.lkv_mla_decode(q, qr, kv, kv[0, 512:], bt, sl, page_size=64,
                                  softmax_scale=0.1, kv_tok_stride=576, rope_tok_stride=576)
    assert out.shape[0] == 0


# ------------------------------------------------- block-table indexing, exact
def test_block_table_one_hot_bit_exact(lkv):
    """q_nope = 0, q_rope[h] = e_{h mod 64}; k_rope is zero except 2^13 at one
    chosen token j*(b, d) per RoPE column d.  Every other score is at least
    340 (natural units) below, so P is exactly one-hot in fp32 and bf16, and
    the output row must equal the bf16 latent row c_{j*} bit for bit."""
    w, x = small_mla(500, B=4, s_q=1, seqlens=[700, 64, 65, 1000], table="fragmented")
    rng = np.random.default_rng(7)
    x["q_nope"][:] = 0
    qr = np.zeros(x["q_rope"].shape, np.float32)
    for h in range(w.h_q):
        qr[:, :, h, h % w.d_rope] = 1.0
    x["q_rope"] = li.to_bf16_bits(qr)
    kv = x["kv"]
    valid = li.valid_slot_mask(x["block_table"], x["seqlens"], w.page_size, x["num_pages"])
    kv[..., w.d_c:][valid] = 0
    target = np.zeros((w.B, w.d_rope), np.int64)
    big = li.to_bf16_bits(np.array([8192.0], np.float32))[0]
    for b in range(w.B):
        L = int(x["seqlens"][b])
        for dd in range(w.d_rope):
            j = int(rng.integers(0, L))
            target[b, dd] = j
            p, s = x["block_table"][b, j // w.page_size], j % w.page_size
            kv[p, s, w.d_c + dd] = big
    note("case one-hot block table")
    d = mla_device_inputs(x, w, torch)
    out, _ = run_mla(lkv, w, d, x=x)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(w.B):
        for h in range(w.h_q):
            j = target[b, h % w.d_rope]
            p, s = x["block_table"][b, j // w.page_size], j % w.page_size
            np.testing.assert_array_equal(got[b, 0, h], kv[p, s, :w.d_c])


def test_page_permutation_and_repeat_bit_identical(lkv):
    w, x = small_mla(510, B=3, s_q=2, seqlens=[500, 130, 64])
    d = mla_device_inputs(x, w, torch)
    o1, l1 = run_mla(lkv, w, d, x=x)
    o1b, l1b = run_mla(lkv, w, d, x=x)
    perm = np.random.default_rng(3).permutation(x["num_pages"])
    inv = np.argsort(perm)
    y = dict(x)
    y["kv"] = x["kv"][perm].copy()
    bt = x["block_table"].copy()
    bt[bt >= 0] = inv[bt[bt >= 0]]
    y["block_table"] = bt
    d2 = mla_device_inputs(y, w, torch)
    o2, l2 = run_mla(lkv, w, d2, x=y)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o1b.view(torch.int16)) and torch.equal(l1, l1b)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# ------------------------------------------------------------------ GQA path
def _gqa_small(seed, *, B=3, h_q=32, n_kv=8, d_h=128, d_rope=0, s_q=1, seqlens=(100, 700, 65),
               causal=True, page=64, cache=""):
    w = li.Workload(name="g", kind="gqa", dtype="bf16", B=len(seqlens), h_q=h_q, s_q=s_q,
                    page_size=page, n_kv=n_kv, d_h=d_h, d_rope=d_rope, seqlens=tuple(seqlens),
                    table="shuffled", causal=causal, scale=1 / math.sqrt(d_h + d_rope),
                    seed=seed, cache=cache)
    return w, li.generate(w)


@pytest.mark.parametrize("h_q,n_kv,d_h,d_rope,s_q,causal,seqlens", [
    (8, 2, 64, 0, 1, True, (100, 700, 65)),
    (16, 4, 32, 8, 2, True, (0, 1, 130, 64)),       # empty and one-token rows
    (8, 1, 128, 16, 3, False, (300, 5, 1000)),      # many tiles per wave
    (32, 8, 16, 0, 1, True, (17, 250))])
def test_fp32_gqa(lkv, oracle, h_q, n_kv, d_h, d_rope, s_q, causal, seqlens):
    """The float32 kernel over separate K and V caches (the value rows are
    staged beside the keys), with and without a shared RoPE key."""
    w = li.Workload(name="g", kind="gqa", dtype="f32", B=len(seqlens), h_q=h_q, s_q=s_q,
                    page_size=16, n_kv=n_kv, d_h=d_h, d_rope=d_rope, seqlens=tuple(seqlens),
                    table="shuffled", causal=causal, scale=1 / math.sqrt(d_h + d_rope),
                    seed=1700 + h_q + d_h)
    x = li.generate(w)
    assert x["q"].dtype == np.float32
    note(f"case fp32 gqa h_q={h_q} n_kv={n_kv} d_h={d_h} d_rope={d_rope} s_q={s_q} causal={causal}")
    out, lse = _run_gqa(lkv, w, x)
    ro, rl = _oracle_gqa(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, f32=True, what="fp32 gqa")


def _run_gqa(lkv, w, x, **kw):
    dev = {k: to_dev(x[k], torch) for k in ("q", "k_cache", "v_cache")}
    qr = to_dev(x["q_rope"], torch) if w.d_rope else None
    kr = to_dev(x["k_rope"], torch) if w.d_rope else None
    return lkv.lkv_gqa_decode(dev["q"], qr, dev["k_cache"], dev["v_cache"], kr,
                              torch.from_numpy(x["block_table"]).cuda(),
                              torch.from_numpy(x["seqlens"]).cuda(), n_kv=w.n_kv,
                              page_size=w.page_size, softmax_scale=w.scale, causal=w.causal,
                              seqlens_host=x["seqlens"], **kw)


def _oracle_gqa(oracle, w, x, rows=None):
    return oracle.gqa_decode(x["q"], x["k_cache"], x["v_cache"], x["block_table"], x["seqlens"],
                             n_kv=w.n_kv, d_h=w.d_h, page_size=w.page_size, scale=w.scale,
                             causal=w.causal, q_rope=x.get("q_rope"), k_rope=x.get("k_rope"),
                             d_rope=w.d_rope, rows=rows)


@pytest.mark.parametrize("h_q,n_kv,d_h,d_rope,s_q,splits,causal", [
    (32, 8, 128, 0, 1, 0, True), (128, 8, 128, 64, 2, 0, True), (128, 8, 128, 64, 2, 7, True),
    (64, 2, 64, 0, 1, 3, True), (16, 16, 256, 0, 1, 0, True), (8, 1, 128, 0, 2, 0, True),
    # GQLA g = 4, s_q = 1; four query tokens (MTP) on g = 8; GQA-2 with 64
    # query heads per KV head (VHA)
    (128, 4, 128, 64, 1, 0, True), (128, 8, 128, 64, 4, 0, True), (128, 2, 128, 0, 1, 0, True),
    # no causal masking among the step's query tokens: every token sees the
    # whole cache, with 16- and 32-row tiles and a split plan
    (128, 8, 128, 64, 2, 0, False), (128, 8, 128, 64, 2, 5, False), (32, 8, 128, 0, 4, 0, False),
    (8, 1, 128, 0, 3, 2, False), (64, 2, 64, 0, 4, 0, False)])
def test_gqa_small(lkv, oracle, h_q, n_kv, d_h, d_rope, s_q, splits, causal):
    w, x = _gqa_small(600 + h_q + d_h + (0 if causal else 11 * s_q), h_q=h_q, n_kv=n_kv, d_h=d_h,
                      d_rope=d_rope, s_q=s_q, causal=causal)
    note(f"case gqa h_q={h_q} n_kv={n_kv} d_h={d_h} d_rope={d_rope} s_q={s_q} splits={splits} "
         f"causal={causal}")
    out, lse = _run_gqa(lkv, w, x, num_splits=splits)
    ro, rl = _oracle_gqa(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what="gqa")


# ------------------------------------------------ expansion and GQLA paths
def _gqla_small(seed, B=2, seqlens=(130, 64)):
    w = li.Workload(name="gqla", kind="gqla", dtype="bf16", B=B, h_q=128, s_q=2, page_size=64,
                    n_lat=1, d_c=512, n_kv=8, d_h=128, d_rope=64, seqlens=tuple(seqlens),
                    table="shuffled", scale=1 / math.sqrt(192), seed=seed)
    return w, li.generate(w)


def _expand_gpu(lkv, w, x, start_pos=None):
    kv = to_dev(x["kv"], torch)
    npg = x["num_pages"]
    k_out = torch.full((npg, w.page_size, w.n_kv, w.d_h), float("nan"), dtype=torch.bfloat16,
                       device="cuda")
    v_out = torch.full_like(k_out, float("nan"))
    sp = None if start_pos is None else torch.from_numpy(start_pos).cuda()
    lkv.lkv_gqla_expand_latent(kv.reshape(-1), to_dev(x["w_uk"], torch), to_dev(x["w_uv"], torch),
                               torch.from_numpy(x["block_table"]).cuda(),
                               torch.from_numpy(x["seqlens"]).cuda(), k_out, v_out,
                               page_size=w.page_size, kv_tok_stride=w.d_c + w.d_rope,
                               start_pos=sp)
    return kv, k_out, v_out


def _w64(x, k):
    return li.bf16_bits_to_f32(x[k]).astype(np.float64)


@pytest.mark.parametrize("g,d_c,d_h,seqlens,page", [
    (8, 512, 128, (130, 64), 64),
    # three groups of 64 (a partial 256-column tile), one group of 256,
    # sequences spanning several 256-token tiles with ragged ends
    (3, 256, 64, (600, 257, 1), 64), (1, 128, 256, (300, 513), 64),
    # latent widths whose count of 32-wide K-chunks is not a multiple of the
    # four-stage ring (2, 6, 14 chunks), pages of 16, 48 and 1000 tokens
    (2, 64, 128, (300, 17), 16), (4, 192, 64, (500, 96, 257), 48),
    (1, 448, 256, (1001, 3), 1000)])
def test_expand_matches_oracle(lkv, oracle, g, d_c, d_h, seqlens, page):
    w = li.Workload(name="gqla", kind="gqla", dtype="bf16", B=len(seqlens), h_q=16 * g, s_q=1,
                    page_size=page, n_lat=1, d_c=d_c, n_kv=g, d_h=d_h, d_rope=64,
                    seqlens=tuple(seqlens), table="shuffled", scale=1 / math.sqrt(d_h + 64),
                    seed=700 + g + d_c)
    x = li.generate(w)
    note(f"case expand g={g} d_c={d_c} d_h={d_h} seqlens={seqlens} page={page}")
    _, k_out, v_out = _expand_gpu(lkv, w, x)
    rk, rv = oracle.expand_latent(x["kv"].reshape(-1), _w64(x, "w_uk"), _w64(x, "w_uv"),
                                  x["block_table"], x["seqlens"], page_size=w.page_size,
                                  num_pages=x["num_pages"], kv_tok_stride=w.d_c + w.d_rope)
    valid = li.valid_slot_mask(x["block_table"], x["seqlens"], w.page_size, x["num_pages"])
    for got, ref in ((from_dev(k_out), rk), (from_dev(v_out), rv)):
        g, r = got[valid], ref[valid]
        # fp32 accumulation, one bf16 rounding: within 2 bf16 ulps of the fp64 value
        tol = 2 * 2.0 ** -8 * np.abs(r) + 1e-6
        assert (np.abs(g - r) <= tol).all(), float(np.abs(g - r).max())
        assert np.isnan(got[~valid]).all(), "rows of invalid tokens were written"


def _expand_gpu_fp8(lkv, w, x, scale):
    kv = to_dev(x["kv"], torch)
    npg = x["num_pages"]
    k8 = torch.full((npg, w.page_size, w.n_kv, w.d_h), 0x7F, dtype=torch.uint8, device="cuda")
    v8 = torch.full_like(k8, 0x7F)
    lkv.lkv_gqla_expand_latent(kv.reshape(-1), to_dev(x["w_uk"], torch), to_dev(x["w_uv"], torch),
                               torch.from_numpy(x["block_table"]).cuda(),
                               torch.from_numpy(x["seqlens"]).cuda(), k8, v8,
                               page_size=w.page_size, kv_tok_stride=w.d_c + w.d_rope,
                               out_fp8=True, out_scale=scale)
    return kv, k8, v8


@pytest.mark.parametrize("g,d_c,d_h,seqlens,scale", [
    (8, 512, 128, (130, 64), 1.0 / 16), (3, 256, 64, (600, 257, 1), 1.0 / 16),
    (1, 128, 256, (300, 513), 1.0 / 16),
    # a scale that is not a power of two: the float32 product with the
    # float32 reciprocal rounds once more (2^-24 relative) before the encoding
    (8, 512, 128, (130, 64), 0.37), (3, 256, 64, (600, 257, 1), 0.37),
    (4, 192, 64, (500, 96, 257), 1.0 / 16)])
def test_expand_fp8_codes(lkv, oracle, g, d_c, d_h, seqlens, scale):
    """8-bit expanded caches: the kernel rounds its float32 result, the
    oracle its fp64 one, so the codes agree except where a value lies within
    float32 accumulation error of a midpoint between two codes -- and there
    the two codes are that midpoint's neighbours."""
    w = li.Workload(name="gqla", kind="gqla", dtype="bf16", B=len(seqlens), h_q=16 * g, s_q=1,
                    page_size=64, n_lat=1, d_c=d_c, n_kv=g, d_h=d_h, d_rope=64,
                    seqlens=tuple(seqlens), table="shuffled", scale=1 / math.sqrt(d_h + 64),
                    seed=720 + g)
    x = li.generate(w)
    note(f"case expand fp8 g={g} d_c={d_c} d_h={d_h} seqlens={seqlens} scale={scale}")
    _, k8, v8 = _expand_gpu_fp8(lkv, w, x, scale)
    rk, rv = oracle.expand_latent(x["kv"].reshape(-1), _w64(x, "w_uk"), _w64(x, "w_uv"),
                                  x["block_table"], x["seqlens"], page_size=w.page_size,
                                  num_pages=x["num_pages"], kv_tok_stride=w.d_c + w.d_rope)
    valid = li.valid_slot_mask(x["block_table"], x["seqlens"], w.page_size, x["num_pages"])
    for got8, ref in ((k8, rk), (v8, rv)):
        got = got8.cpu().numpy()
        xv = ref[valid] / scale
        want = oracle.e4m3_from_f64(xv)
        gv = got[valid]
        diff = gv != want
        assert diff.mean() < 1e-2, float(diff.mean())
        if diff.any():
            a, b = oracle.e4m3_to_f64(gv[diff]), oracle.e4m3_to_f64(want[diff])
            mid = (a + b) / 2
            assert np.all(np.abs(xv[diff] - mid) <= 2e-4 * (np.abs(xv[diff]) + 1)), \
                float(np.max(np.abs(xv[diff] - mid)))
        assert (got[~valid] == 0x7F).all(), "rows of invalid tokens were written"


def test_expand_fp8_rounding_is_exact(lkv, oracle):
    """The kernel's E4M3 rounding on exactly known values: W_UK = I and
    W_UV = -I make K = c and V = -c exactly, so with out_scale 1 the codes
    must equal the oracle's encoding of c bit for bit -- every code's value,
    every midpoint between adjacent codes (ties to the even code), points an
    eighth of a step either side, magnitudes past 448, subnormal ties."""
    dec, enc = oracle.e4m3_to_f64, oracle.e4m3_from_f64
    mags = dec(np.arange(0x7F, dtype=np.uint8))
    mid = (mags[:-1] + mags[1:]) / 2
    step = mags[1:] - mags[:-1]
    vals = np.concatenate([mags, mid, mid - step / 8, mid + step / 8,
                           [448.0, 456.0, 464.0, 472.0, 480.0, 1000.0, 2.0 ** 20,
                            2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -12, 0.0]])
    assert np.array_equal(li.bf16_bits_to_f32(li.to_bf16_bits(vals)), vals.astype(np.float32))
    d = 128
    w = li.Workload(name="gqla", kind="gqla", dtype="bf16", B=1, h_q=16, s_q=1, page_size=64,
                    n_lat=1, d_c=d, n_kv=1, d_h=d, d_rope=64, seqlens=(64,), table="shuffled",
                    scale=1 / math.sqrt(d + 64), seed=1700)
    x = li.generate(w)
    cells = np.zeros(64 * d)
    cells[:vals.size] = vals
    cells = cells.reshape(64, d)
    page = x["block_table"][0, 0]
    x["kv"][page, :, :d] = li.to_bf16_bits(cells)
    eye = np.eye(d)[None]
    x["w_uk"], x["w_uv"] = li.to_bf16_bits(eye), li.to_bf16_bits(-eye)
    note("case expand fp8 exact rounding")
    _, k8, v8 = _expand_gpu_fp8(lkv, w, x, 1.0)
    got_k = k8.cpu().numpy()[page, :, 0, :]
    got_v = v8.cpu().numpy()[page, :, 0, :]
    assert np.array_equal(got_k, enc(cells)), np.argwhere(got_k != enc(cells))[:5]
    # V = c (-I) sums products from +0, so an exact zero is +0 (as in the
    # oracle's fp64 expansion); + 0.0 turns numpy's -0.0 into +0.0
    want_v = enc(-cells + 0.0)
    assert np.array_equal(got_v, want_v), np.argwhere(got_v != want_v)[:5]


def test_expand_nan_latent_gives_nan(lkv, oracle):
    """A NaN in a valid token's latent row makes that token's expanded K and V
    NaN: bf16 NaN on the bf16 path, the E4M3 NaN code (S.1111.111) on the
    8-bit path -- never a finite (saturated) value."""
    w, x = _gqla_small(1650, seqlens=(130, 64))
    b, j = 0, 77
    page, slot = x["block_table"][b, j // w.page_size], j % w.page_size
    x["kv"][page, slot, : w.d_c] = li.BF16_NAN
    note("case expand NaN latent row")
    _, k_out, v_out = _expand_gpu(lkv, w, x)
    _, k8, v8 = _expand_gpu_fp8(lkv, w, x, 1.0 / 16)
    for t in (k_out, v_out):
        assert np.isnan(from_dev(t)[page, slot]).all()
    for t in (k8, v8):
        codes = t.cpu().numpy()
        assert ((codes[page, slot] & 0x7F) == 0x7F).all()
        others = np.ones(codes.shape[:2], bool)
        others[page, slot] = False
        valid = li.valid_slot_mask(x["block_table"], x["seqlens"], w.page_size, x["num_pages"])
        assert ((codes[others & valid] & 0x7F) != 0x7F).all()


def test_gqla_fp8_expanded_cache_end_to_end(lkv, oracle):
    """The grouped path over 8-bit caches written by the library: expansion
    into E4M3 K/V and the RoPE key appended as codes of the same scale (every
    position of each sequence in one append of s_q = the longest length),
    then grouped decode reading them, against the oracle's decode over its
    own expansion quantised by its own encoder."""
    scale = 1.0 / 16
    w, x = _gqla_small(1600, seqlens=(130, 64))
    note("case GQLA over 8-bit expanded caches")
    _, k8, v8 = _expand_gpu_fp8(lkv, w, x, scale)
    P, bt, lens = w.page_size, x["block_table"], x["seqlens"]
    S = int(lens.max())
    rope = x["kv"][..., w.d_c:]
    new = np.zeros((w.B, S, w.d_rope), np.uint16)
    for b, L in enumerate(lens):
        for t in range(S):
            j = int(L) - S + t
            if j >= 0:
                new[b, t] = rope[bt[b, j // P], j % P]
    rope8 = torch.full((x["num_pages"] * P * w.d_rope,), 0x7F, dtype=torch.uint8, device="cuda")
    lkv.lkv_append_tokens(to_dev(new, torch), rope8, torch.from_numpy(bt).cuda(),
                          torch.from_numpy(lens).cuda(), page_size=P, out_fp8=True, out_scale=scale)
    rope_codes = rope8.cpu().numpy().reshape(x["num_pages"], P, w.d_rope)
    valid = li.valid_slot_mask(bt, lens, P, x["num_pages"])
    want = oracle.e4m3_from_f64(li.bf16_bits_to_f32(rope).astype(np.float64) / scale)
    assert np.array_equal(rope_codes[valid], want[valid])
    out, lse = lkv.lkv_gqa_decode(to_dev(x["q_nope_h"], torch), to_dev(x["q_rope"], torch), k8, v8,
                                  rope8, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                                  n_kv=w.n_kv, page_size=P, softmax_scale=w.scale,
                                  rope_tok_stride=w.d_rope, kv_fp8=True, kv_scale=scale)
    rk, rv = oracle.expand_latent(x["kv"].reshape(-1), _w64(x, "w_uk"), _w64(x, "w_uv"),
                                  x["block_table"], x["seqlens"], page_size=w.page_size,
                                  num_pages=x["num_pages"], kv_tok_stride=w.d_c + w.d_rope)
    kq = oracle.e4m3_to_f64(oracle.e4m3_from_f64(rk / scale), scale)
    vq = oracle.e4m3_to_f64(oracle.e4m3_from_f64(rv / scale), scale)
    rq = oracle.e4m3_to_f64(rope_codes, scale)
    ro, rl = oracle.gqa_decode(_w64(x, "q_nope_h"), np.nan_to_num(kq), np.nan_to_num(vq),
                               x["block_table"], x["seqlens"], n_kv=w.n_kv, d_h=w.d_h,
                               page_size=w.page_size, scale=w.scale, causal=w.causal,
                               q_rope=_w64(x, "q_rope"), k_rope=np.nan_to_num(rq),
                               d_rope=w.d_rope)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what="GQLA fp8 expanded")


def test_expand_start_pos(lkv):
    w, x = _gqla_small(701)
    sp = np.array([70, 0], np.int32)
    _, k_out, _ = _expand_gpu(lkv, w, x, start_pos=sp)
    k = from_dev(k_out)
    bt = x["block_table"]
    for j in (0, 69):
        assert np.isnan(k[bt[0, j // 64], j % 64]).all()
    assert np.isfinite(k[bt[0, 70 // 64], 70 % 64]).all()
    assert np.isfinite(k[bt[1, 0], 0]).all()


def test_gqla_grouped_and_absorbed_paths(lkv, oracle):
    """GQLA section 2: the same weights give two paths.  GPU grouped path
    (expansion kernel, then grouped decode over the bf16 K/V) and GPU
    absorbed path (latent decode with q' = W_UK q, then W_UV) both match the
    oracle's grouped path, and each other."""
    w, x = _gqla_small(702)
    note("case gqla paths")
    kv, k_out, v_out = _expand_gpu(lkv, w, x)
    q_h = li.bf16_bits_to_f32(x["q_nope_h"]).astype(np.float64)
    q_r = x["q_rope"]
    flat = kv.reshape(-1)
    out_g, lse_g = lkv.lkv_gqa_decode(to_dev(x["q_nope_h"], torch), to_dev(q_r, torch), k_out,
                                      v_out, flat[w.d_c:], torch.from_numpy(x["block_table"]).cuda(),
                                      torch.from_numpy(x["seqlens"]).cuda(), n_kv=w.n_kv,
                                      page_size=w.page_size, softmax_scale=w.scale,
                                      rope_tok_stride=w.d_c + w.d_rope, seqlens_host=x["seqlens"])
    wuk, wuv = _w64(x, "w_uk"), _w64(x, "w_uv")
    rk, rv = oracle.expand_latent(x["kv"].reshape(-1), wuk, wuv, x["block_table"], x["seqlens"],
                                  page_size=w.page_size, num_pages=x["num_pages"],
                                  kv_tok_stride=w.d_c + w.d_rope)
    rk, rv = np.nan_to_num(rk), np.nan_to_num(rv)
    kv64 = li.bf16_bits_to_f32(x["kv"]).astype(np.float64)
    ro, rl = oracle.gqa_decode(q_h, rk, rv, x["block_table"], x["seqlens"], n_kv=w.n_kv, d_h=w.d_h,
                               page_size=w.page_size, scale=w.scale,
                               q_rope=li.bf16_bits_to_f32(q_r).astype(np.float64),
                               k_rope=np.nan_to_num(kv64[..., w.d_c:]).copy(), d_rope=w.d_rope)
    assert_close(from_dev(out_g), ro, from_dev(lse_g), rl, what="gqla grouped (GPU) vs oracle")
    # absorbed path: q' from the oracle's absorb step, rounded to bf16 as the input
    qa = oracle.absorb_query(q_h, wuk)
    qa_bits = li.to_bf16_bits(qa.astype(np.float32))
    dev = dict(q_nope=to_dev(qa_bits, torch), q_rope=to_dev(q_r, torch))
    out_a, lse_a = lkv.lkv_mla_decode(dev["q_nope"], dev["q_rope"], flat, flat[w.d_c:],
                                      torch.from_numpy(x["block_table"]).cuda(),
                                      torch.from_numpy(x["seqlens"]).cuda(), page_size=w.page_size,
                                      softmax_scale=w.scale, kv_tok_stride=w.d_c + w.d_rope,
                                      rope_tok_stride=w.d_c + w.d_rope, seqlens_host=x["seqlens"])
    o_abs = oracle.up_project(from_dev(out_a), wuv)
    assert_close(o_abs, ro, from_dev(lse_a), rl, what="gqla absorbed (GPU) + W_UV vs oracle grouped")


# ------------------------------------------- steps either side of decode
@pytest.mark.parametrize("B,s_q,h_q,n_w,d_c,d_h", [
    (3, 2, 16, 16, 512, 128),    # per-head weights (MLA)
    (2, 2, 128, 8, 512, 128),    # group-indexed weights (GQLA)
    (5, 1, 12, 3, 256, 64)])     # row count not a multiple of the 64-row tile
def test_absorb_and_up_project_match_oracle(lkv, oracle, B, s_q, h_q, n_w, d_c, d_h):
    rng = np.random.default_rng(900 + h_q + d_c)
    q = li.to_bf16_bits(rng.standard_normal((B, s_q, h_q, d_h)).astype(np.float32))
    o = li.to_bf16_bits(rng.standard_normal((B, s_q, h_q, d_c)).astype(np.float32))
    w = li.to_bf16_bits((rng.standard_normal((n_w, d_c, d_h)) / math.sqrt(d_c)).astype(np.float32))
    note(f"case projections B={B} s_q={s_q} h_q={h_q} n_w={n_w} d_c={d_c} d_h={d_h}")
    f = lambda a: li.bf16_bits_to_f32(a).astype(np.float64)
    for name, x, ref_fn in (("absorb", q, oracle.absorb_query), ("up", o, oracle.up_project)):
        fn = lkv.lkv_absorb_query if name == "absorb" else lkv.lkv_up_project
        got = from_dev(fn(to_dev(x, torch), to_dev(w, torch)))
        ref = ref_fn(f(x), f(w))
        mag = ref_fn(np.abs(f(x)), np.abs(f(w)))  # sum of |terms| per output
        # one bf16 rounding of the output plus float32 accumulation
        tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -18 * mag + 1e-30
        err = np.abs(got - ref)
        note(f"  {name}: max err/tol {float((err / tol).max()):.3f}")
        assert (err <= tol).all(), name


def test_append_tokens_bit_exact(lkv, oracle):
    w, x = small_mla(910, B=3, s_q=2, seqlens=[130, 2, 64])
    width = w.n_lat * w.d_c + w.d_rope
    rng = np.random.default_rng(911)
    src = li.to_bf16_bits(rng.standard_normal((w.B, w.s_q, width)).astype(np.float32))
    kv = to_dev(x["kv"], torch)
    note("case append")
    lkv.lkv_append_tokens(to_dev(src, torch), kv, torch.from_numpy(x["block_table"]).cuda(),
                          torch.from_numpy(x["seqlens"]).cuda(), page_size=w.page_size)
    torch.cuda.synchronize()
    got = kv.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
    ref = oracle.append_tokens(src, x["kv"], x["block_table"], x["seqlens"],
                               page_size=w.page_size, tok_stride=width)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16).reshape(-1))


@pytest.mark.parametrize("scale", [1.0 / 16, 0.37])
def test_append_tokens_fp8_bit_exact(lkv, oracle, scale):
    """8-bit cache write: each bf16 value x becomes the code of fl32(x *
    fl32(1 / scale)).  Both sides round that float32 product (the oracle's
    encoder takes it exactly), so the codes agree bit for bit -- special
    values included (NaN, infinities, magnitudes past 448, subnormals); rows
    of negative positions and untouched slots keep their bytes."""
    rng = np.random.default_rng(912)
    B, s_q, width, P = 3, 5, 64 + 32, 16
    seqlens = np.array([40, 3, 17], np.int32)
    npages = 12
    bt = rng.permutation(npages)[: B * 4].reshape(B, 4).astype(np.int32)
    x = (rng.standard_normal((B, s_q, width)) * 8).astype(np.float32)
    x[0, 0, :6] = [np.nan, np.inf, -np.inf, 1000.0, -449.0, 2.0 ** -12]
    x[1, 4, :4] = [-0.0, 2.0 ** -10, -(2.0 ** -9) * 1.5, 0.0]
    src = li.to_bf16_bits(x)
    cache0 = rng.integers(0, 256, (npages * P, width), dtype=np.uint8)
    cache = torch.from_numpy(cache0.copy()).cuda()
    note(f"case append fp8 scale={scale}")
    lkv.lkv_append_tokens(to_dev(src, torch), cache, torch.from_numpy(bt).cuda(),
                          torch.from_numpy(seqlens).cuda(), page_size=P, out_fp8=True,
                          out_scale=scale)
    torch.cuda.synchronize()
    got = cache.cpu().numpy().reshape(-1)
    inv = np.float32(1) / np.float32(scale)
    prod = (li.bf16_bits_to_f32(src) * inv).astype(np.float32)
    ref = oracle.append_tokens(oracle.e4m3_from_f64(prod.astype(np.float64)), cache0, bt,
                               seqlens, page_size=P, tok_stride=width)
    assert np.array_equal(got, ref.reshape(-1))


def test_decode_layer_on_gpu(lkv, oracle):
    """The whole absorbed decode layer on the GPU -- W_UK into the query,
    the step's new tokens into the cache, latent decode, W_UV on the output
    -- against the oracle's grouped path on the same weights."""
    w, x = _gqla_small(920)
    width = w.d_c + w.d_rope
    P = w.page_size
    # the cache as it stood before this step: the last s_q tokens of each
    # sequence are absent (NaN) and come in through the append
    kv0 = x["kv"].copy()
    for b, L in enumerate(x["seqlens"]):
        for j in range(int(L) - w.s_q, int(L)):
            kv0[x["block_table"][b, j // P], j % P] = li.BF16_NAN
    new = np.stack([np.stack([x["kv"][x["block_table"][b, j // P], j % P]
                              for j in range(int(L) - w.s_q, int(L))])
                    for b, L in enumerate(x["seqlens"])])
    kv = to_dev(kv0, torch)
    flat = kv.reshape(-1)
    bt, sl = torch.from_numpy(x["block_table"]).cuda(), torch.from_numpy(x["seqlens"]).cuda()
    note("case decode layer")
    lkv.lkv_append_tokens(to_dev(new, torch), kv, bt, sl, page_size=P)
    q_abs = lkv.lkv_absorb_query(to_dev(x["q_nope_h"], torch), to_dev(x["w_uk"], torch))
    out, lse = lkv.lkv_mla_decode(q_abs, to_dev(x["q_rope"], torch), flat, flat[w.d_c:], bt, sl,
                                  page_size=P, softmax_scale=w.scale, kv_tok_stride=width,
                                  rope_tok_stride=width, seqlens_host=x["seqlens"])
    o = lkv.lkv_up_project(out, to_dev(x["w_uv"], torch))
    wuk, wuv = _w64(x, "w_uk"), _w64(x, "w_uv")
    rk, rv = oracle.expand_latent(x["kv"].reshape(-1), wuk, wuv, x["block_table"], x["seqlens"],
                                  page_size=P, num_pages=x["num_pages"], kv_tok_stride=width)
    kv64 = li.bf16_bits_to_f32(x["kv"]).astype(np.float64)
    ro, rl = oracle.gqa_decode(_w64(x, "q_nope_h"), np.nan_to_num(rk), np.nan_to_num(rv),
                               x["block_table"], x["seqlens"], n_kv=w.n_kv, d_h=w.d_h,
                               page_size=P, scale=w.scale, q_rope=_w64(x, "q_rope"),
                               k_rope=np.nan_to_num(kv64[..., w.d_c:]).copy(), d_rope=w.d_rope)
    assert_close(from_dev(o), ro, from_dev(lse), rl, what="decode layer (GPU) vs oracle grouped")


# ------------------------------------------------------------ split combine
def test_split_combine_entry_point(lkv, oracle):
    rng = np.random.default_rng(800)
    B, s_q, h_q, dv = 4, 2, 16, 512
    counts = [3, 0, 1, 5]
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(offs[-1])
    o_part = rng.standard_normal((n, s_q, h_q, dv)).astype(np.float32)
    lse_part = (rng.standard_normal((n, s_q, h_q)) * 3).astype(np.float32)
    lse_part[0, 0, :4] = -np.inf          # an empty split inside a sequence
    lse_part[1:3, 1, 2] = -np.inf
    ro, rl = oracle.lse_combine(o_part.astype(np.float64), lse_part.astype(np.float64), offs)
    for dt in (torch.float32, torch.bfloat16):
        note(f"case combine {dt}")
        out, lse = lkv.lkv_split_combine(torch.from_numpy(o_part).cuda(),
                                         torch.from_numpy(lse_part).cuda(),
                                         torch.from_numpy(offs).cuda(), dtype=dt)
        assert_close(from_dev(out), ro, from_dev(lse), rl, f32=dt == torch.float32,
                     what=f"combine {dt}")


# ------------------------------------------------------------ 8-bit caches
# The caches hold OCP E4M3 codes of value / kv_scale; the oracle sees the
# dequantised values (float32, exact) and float32 copies of the bf16 queries.
GQA_KEYS = ["k_cache", "v_cache"]


def _fp8(w):
    return dict(kv_fp8=True, kv_scale=w.kv_scale)


@pytest.mark.parametrize("h_q,n_kv,d_h,d_rope,s_q,splits,page,seqlens,causal", [
    (32, 8, 128, 0, 1, 0, 64, (100, 700, 65), True),
    (128, 8, 128, 64, 2, 0, 64, (100, 700, 65), True),     # GQLA grouped, g = 8
    (128, 8, 128, 64, 2, 7, 64, (100, 700, 65), True),
    (128, 2, 128, 0, 1, 0, 64, (0, 1, 130, 64), True),    # GQA-2; empty and 1-token rows
    (8, 1, 128, 0, 2, 3, 48, (100, 700, 65), True),       # general pages
    (32, 8, 128, 64, 1, 0, 16, (333, 64, 1000), True),
    # GQLA grouped with no causal masking among the step's two query tokens
    (128, 8, 128, 64, 2, 0, 64, (100, 700, 65), False),
    (128, 8, 128, 64, 2, 3, 48, (2, 700, 129), False)])
def test_gqa_fp8(lkv, oracle, h_q, n_kv, d_h, d_rope, s_q, splits, page, seqlens, causal):
    w, x = _gqa_small(900 + h_q + page + splits + (0 if causal else 17), h_q=h_q, n_kv=n_kv,
                      d_h=d_h, d_rope=d_rope, s_q=s_q, page=page, seqlens=seqlens, cache="fp8",
                      causal=causal)
    assert x["k_cache"].dtype == np.uint8
    note(f"case gqa fp8 h_q={h_q} n_kv={n_kv} d_rope={d_rope} s_q={s_q} splits={splits} "
         f"page={page} seqlens={seqlens} causal={causal}")
    out, lse = _run_gqa(lkv, w, x, num_splits=splits, **_fp8(w))
    keys = GQA_KEYS + (["k_rope"] if d_rope else [])
    y = dequantised(oracle, x, keys, ["q"] + (["q_rope"] if d_rope else []))
    ro, rl = _oracle_gqa(oracle, w, y)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what="gqa fp8")


@pytest.mark.parametrize("h_q,n_lat,d_c,s_q,splits,page,seqlens,causal", [
    (16, 1, 512, 1, 0, 64, (70, 600, 129, 1), True),      # few-head MLA
    (128, 1, 512, 1, 0, 64, (70, 600, 129, 1), True),     # many-row MLA
    (128, 1, 512, 2, 5, 48, (70, 600, 129, 2), True),
    (32, 2, 256, 1, 0, 64, (0, 300, 1000), True),         # GLA-2
    (32, 2, 256, 2, 3, 32, (64, 300, 1000), True),
    (32, 8, 128, 1, 0, 64, (500, 65, 128), True),         # GTA
    (128, 2, 256, 1, 0, 64, (70, 600, 129), True),        # GLA-2, many rows per latent head
    (128, 2, 256, 2, 3, 48, (70, 600, 129), True),
    # no causal masking among the query tokens: GLA-2 on the row-tiled kernel,
    # and many-row MLA
    (32, 2, 256, 2, 0, 64, (2, 300, 1000), False),
    (128, 1, 512, 2, 3, 64, (70, 600, 129), False)])
def test_mla_fp8(lkv, oracle, h_q, n_lat, d_c, s_q, splits, page, seqlens, causal):
    w, x = small_mla(950 + h_q + d_c + s_q + page + (0 if causal else 5), h_q=h_q, n_lat=n_lat,
                     d_c=d_c, s_q=s_q, page=page, seqlens=seqlens, cache="fp8", causal=causal)
    assert x["kv"].dtype == np.uint8
    note(f"case mla fp8 h_q={h_q} n_lat={n_lat} d_c={d_c} s_q={s_q} splits={splits} page={page} "
         f"seqlens={seqlens} causal={causal}")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d, x=x, num_splits=splits, **_fp8(w))
    ro, rl = oracle_mla(oracle, w, dequantised(oracle, x, ["kv"], ["q_nope", "q_rope"]))
    assert_close(from_dev(out), ro, from_dev(lse), rl, what="mla fp8")


@pytest.mark.parametrize("d_c,splits", [(512, 0), (256, 5)])
def test_mla_fp8_many_rows_without_rope(lkv, oracle, d_c, splits):
    """The many-row kernel's 8-bit instantiations with no RoPE key."""
    w, x = small_mla(970 + d_c + splits, h_q=128, d_c=d_c, d_rope=0, seqlens=(70, 600, 129),
                     cache="fp8")
    note(f"case mla fp8 d_c={d_c} d_rope=0 splits={splits}")
    d = mla_device_inputs(x, w, torch)
    out, lse = lkv.lkv_mla_decode(d["q_nope"], None, d["c_kv"], None, d["block_table"],
                                  d["seqlens"], page_size=w.page_size, softmax_scale=w.scale,
                                  causal=w.causal, kv_tok_stride=d["kv_tok_stride"],
                                  num_splits=splits, **_fp8(w))
    ro, rl = oracle_mla(oracle, w, dequantised(oracle, x, ["kv"], ["q_nope", "q_rope"]))
    assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"mla fp8 d_c={d_c} no rope")


@pytest.mark.parametrize("kind", ["gqa", "gla2", "mla16"])
def test_fp8_equals_bf16_of_dequantised_cache(lkv, oracle, kind):
    """With a power-of-two kv_scale every scaling is exact, so the 8-bit path
    must give the bits of the bf16 path over the dequantised cache (same
    kernel, same split plan)."""
    if kind == "gqa":
        w, x = _gqa_small(990, h_q=128, n_kv=8, d_rope=64, s_q=2, cache="fp8")
        keys = GQA_KEYS + ["k_rope"]
    else:
        h_q, n_lat, d_c = (32, 2, 256) if kind == "gla2" else (16, 1, 512)
        w, x = small_mla(991, h_q=h_q, n_lat=n_lat, d_c=d_c, seqlens=(70, 600, 129), cache="fp8")
        keys = ["kv"]
    note(f"case fp8 == bf16 of dequantised cache, {kind}")
    lut = li.to_bf16_bits(oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8), w.kv_scale))
    xb = dict(x)
    for k in keys:
        xb[k] = lut[x[k]]
    if kind == "gqa":
        o8, l8 = _run_gqa(lkv, w, x, num_splits=4, **_fp8(w))
        ob, lb = _run_gqa(lkv, w, xb, num_splits=4)
    else:
        o8, l8 = run_mla(lkv, w, mla_device_inputs(x, w, torch), x=x, num_splits=4, **_fp8(w))
        ob, lb = run_mla(lkv, w, mla_device_inputs(xb, w, torch), x=xb, num_splits=4)
    torch.cuda.synchronize()
    assert torch.equal(o8.view(torch.int16), ob.view(torch.int16))
    assert torch.equal(l8, lb)


# ------------------------------------------------- every compiled instantiation
# (key width, RoPE width, value width, latent is the value) of the row-tiled
# kernel, bf16 and 8-bit; each at 16 and at 32 query rows per KV/latent head
ROW_TILED = [(512, 64, 512, True), (256, 64, 256, True), (128, 64, 128, True),
             (512, 0, 512, True), (128, 64, 128, False), (128, 0, 128, False),
             (64, 0, 64, False), (256, 0, 256, False)]
ROW_TILED_F8 = [(512, 64, 512, True), (256, 64, 256, True), (128, 64, 128, True),
                (128, 64, 128, False), (128, 0, 128, False)]
INSTANTIATIONS = ([(v, rows, "") for v in ROW_TILED for rows in (16, 32)]
                  + [(v, rows, "fp8") for v in ROW_TILED_F8 for rows in (16, 32)]
                  + [((dk, dr, dk, True), 64, c) for dk in (512, 256) for dr in (64, 0)
                     for c in ("", "fp8")])


@pytest.mark.parametrize("widths,rows,cache", INSTANTIATIONS,
                         ids=[f"{v[0]}+{v[1]}{'-latent' if v[3] else '-grouped'}-rows{r}{'-' + c if c else ''}"
                              for v, r, c in INSTANTIATIONS])
def test_every_instantiation(lkv, oracle, widths, rows, cache):
    """Each compiled kernel instantiation once, at a small ragged size:
    latent ones through lkv_mla_decode (one latent head; 64 rows select the
    many-row kernel), grouped ones through lkv_gqa_decode (two KV heads)."""
    dk, dr, dv, latent = widths
    seed = 1400 + dk + dr + rows + (7 if cache else 0) + (3 if latent else 0)
    note(f"case instantiation {widths} rows={rows} cache={cache or 'bf16'}")
    q8 = {}
    if latent:
        w, x = small_mla(seed, h_q=rows, d_c=dk, d_rope=dr, seqlens=(70, 200, 1), cache=cache)
        if cache:
            q8 = _fp8(w)
        d = mla_device_inputs(x, w, torch)
        out, lse = lkv.lkv_mla_decode(d["q_nope"], d["q_rope"] if dr else None, d["c_kv"],
                                      d["k_rope"] if dr else None, d["block_table"], d["seqlens"],
                                      page_size=w.page_size, softmax_scale=w.scale,
                                      causal=w.causal, kv_tok_stride=d["kv_tok_stride"],
                                      rope_tok_stride=d["rope_tok_stride"] if dr else None, **q8)
        y = dequantised(oracle, x, ["kv"], ["q_nope", "q_rope"]) if cache else x
        ro, rl = oracle_mla(oracle, w, y)
    else:
        w, x = _gqa_small(seed, h_q=2 * rows, n_kv=2, d_h=dk, d_rope=dr, seqlens=(70, 200, 1),
                          cache=cache)
        if cache:
            q8 = _fp8(w)
        out, lse = _run_gqa(lkv, w, x, **q8)
        keys = GQA_KEYS + (["k_rope"] if dr else [])
        y = dequantised(oracle, x, keys, ["q"] + (["q_rope"] if dr else [])) if cache else x
        ro, rl = _oracle_gqa(oracle, w, y)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"{widths} rows={rows} {cache}")


# ------------------------------------------------------------ graph capture
def test_decode_calls_replay_under_a_hip_graph(lkv):
    """A split MLA call (attention kernel + combine) and a GQA call captured
    in one graph: every replay, each after eager calls on other inputs and a
    synchronisation, matches the eager result bit for bit."""
    w, x = small_mla(1500, h_q=128, seqlens=(300, 1000, 64))
    d = mla_device_inputs(x, w, torch)
    wg, xg = _gqa_small(1501, h_q=32, n_kv=8, seqlens=(300, 1000, 64))
    w2, x2 = small_mla(1502, h_q=128, seqlens=(200, 700, 90))
    d2 = mla_device_inputs(x2, w2, torch)
    s = torch.cuda.Stream()
    ws = torch.empty(lkv.lkv_mla_decode_workspace_size(
        d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["block_table"], d["seqlens"],
        page_size=w.page_size, softmax_scale=w.scale, kv_tok_stride=d["kv_tok_stride"],
        rope_tok_stride=d["rope_tok_stride"], num_splits=7), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q_nope"])
    lse = torch.empty(d["q_nope"].shape[:3], dtype=torch.float32, device="cuda")
    gq = {k: to_dev(xg[k], torch) for k in ("q", "k_cache", "v_cache")}
    gbt, gsl = torch.from_numpy(xg["block_table"]).cuda(), torch.from_numpy(xg["seqlens"]).cuda()
    gout = torch.empty_like(gq["q"])
    gws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")

    def step():
        lkv.lkv_mla_decode(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"], d["block_table"],
                           d["seqlens"], page_size=w.page_size, softmax_scale=w.scale,
                           kv_tok_stride=d["kv_tok_stride"], rope_tok_stride=d["rope_tok_stride"],
                           num_splits=7, seqlens_host=x["seqlens"], out=out, lse=lse,
                           workspace=ws, stream=s)
        lkv.lkv_gqa_decode(gq["q"], None, gq["k_cache"], gq["v_cache"], None, gbt, gsl,
                           n_kv=wg.n_kv, page_size=wg.page_size, softmax_scale=wg.scale,
                           out=gout, workspace=gws, stream=s)

    note("case graph capture: eager reference")
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref_o, ref_l, ref_g = out.clone(), lse.clone(), gout.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        # eager work on other inputs between replays
        run_mla(lkv, w2, d2, x=x2, num_splits=5)
        out.zero_()
        lse.zero_()
        gout.zero_()
        torch.cuda.synchronize()
        note(f"case graph capture: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), r
        assert torch.equal(lse, ref_l), r
        assert torch.equal(gout.view(torch.int16), ref_g.view(torch.int16)), r


def test_default_workspace_per_stream(lkv):
    """Calls that pass no workspace use a cached buffer per (device, stream):
    decodes on two streams at once, with plans that need more workspace
    call after call, give the same bits as the same calls one at a time
    with their own workspaces."""
    cases = []
    for i, (B, splits) in enumerate([(2, 3), (4, 7), (8, 16), (16, 40)]):
        w, x = small_mla(2000 + i, B=B, seqlens=[300 + 97 * j for j in range(B)], table="shuffled")
        cases.append((w, x, mla_device_inputs(x, w, torch), splits))
    refs = []
    for w, x, d, splits in cases:
        need = lkv.lkv_mla_decode_workspace_size(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"],
                                                 d["block_table"], d["seqlens"], n_latent=w.n_lat,
                                                 page_size=w.page_size, softmax_scale=w.scale,
                                                 causal=w.causal, kv_tok_stride=d["kv_tok_stride"],
                                                 rope_tok_stride=d["rope_tok_stride"],
                                                 num_splits=splits)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        o, l = run_mla(lkv, w, d, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        refs.append((o.clone(), l.clone()))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    got = []
    note("case default workspace on two streams")
    for r in range(2):
        for i in range(len(cases)):
            for s, j in ((s1, i), (s2, len(cases) - 1 - i)):
                w, x, d, splits = cases[j]
                with torch.cuda.stream(s):
                    got.append((j, *run_mla(lkv, w, d, num_splits=splits)))
    torch.cuda.synchronize()
    for j, o, l in got:
        assert torch.equal(o.view(torch.int16), refs[j][0].view(torch.int16)), j
        assert torch.equal(l, refs[j][1]), j
    keys = {k for k in lkv._workspaces if k[1] in (s1.cuda_stream, s2.cuda_stream)}
    assert len(keys) == 2


# ----------------------------------------------------- softmax normalisation
def _pages_of(x, b, page):
    L = int(x["seqlens"][b])
    return x["block_table"][b, : (L + page - 1) // page]


@pytest.mark.parametrize("kind,h_q,splits", [("mla", 128, 0), ("mla", 128, 7), ("mla", 16, 0),
                                             ("mla", 16, 5), ("gqa", 32, 0), ("gqa", 32, 7)])
def test_constant_value_rows_give_that_value(lkv, kind, h_q, splits):
    """When every cached value row of a sequence is the same vector v, the
    weights of any row sum to one, so the output is v whatever the scores:
    a missed rescale of O or of the row sum when the running maximum moves,
    a wrong share weight in the combine, or a dropped tile would show.
    Queries are scaled by 8 (exact) so that scores spread and the reference
    maximum moves.  The row sum adds unrounded probabilities while P V uses
    their bf16 values, so the check allows one bf16 ulp."""
    rng = np.random.default_rng(1300 + h_q + splits)
    seqlens = (300, 1000, 64)
    if kind == "mla":
        w, x = small_mla(1301 + h_q + splits, h_q=h_q, seqlens=seqlens)
        width = w.d_c
    else:
        w, x = _gqa_small(1302 + splits, h_q=h_q, n_kv=8, seqlens=seqlens)
        width = w.d_h
    v = li.to_bf16_bits(rng.standard_normal((w.B, w.n_kv if kind == "gqa" else 1, width)))
    for b in range(w.B):
        pages = _pages_of(x, b, w.page_size)
        if kind == "mla":
            x["kv"][pages, :, : w.d_c] = v[b, 0]
        else:
            x["v_cache"][pages] = v[b]
    for k in ("q_nope", "q_rope", "q"):
        if k in x:
            x[k] = li.to_bf16_bits(8.0 * li.bf16_bits_to_f32(x[k]))
    note(f"case constant value rows {kind} h_q={h_q} splits={splits}")
    if kind == "mla":
        out, _ = run_mla(lkv, w, mla_device_inputs(x, w, torch), x=x, num_splits=splits)
    else:
        out, _ = _run_gqa(lkv, w, x, num_splits=splits)
    got = from_dev(out)                                   # [B, s_q, h_q, width]
    hpk = h_q // (w.n_kv if kind == "gqa" else 1)
    want = li.bf16_bits_to_f32(v)[:, np.arange(h_q) // hpk]  # [B, h_q, width]
    want = np.broadcast_to(want[:, None], got.shape)
    assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + 1e-30), \
        float(np.max(np.abs(got - want) / (np.abs(want) + 1e-30)))


def _scale_keys_along_sequence(x, w, kind, direction):
    """Multiply a key-only part of cached token j of every sequence by a
    factor that grows along the sequence (or shrinks, falling), rounded back
    to bf16, leaving the values as they are.  MLA: the shared RoPE key, by 1
    to 32 (the latent is also the value); GQA: the key rows, by 1 to 8."""
    top = 32.0 if kind == "mla" else 8.0
    for b in range(w.B):
        L = int(x["seqlens"][b])
        if L == 0:
            continue
        j = np.arange(L)
        f = 1.0 + (top - 1.0) * j / max(L - 1, 1)
        if direction == "fall":
            f = f[::-1]
        pages = x["block_table"][b, j // w.page_size]
        slots = j % w.page_size
        if kind == "mla":
            c0 = w.n_lat * w.d_c
            rows = li.bf16_bits_to_f32(x["kv"][pages, slots, c0:])
            x["kv"][pages, slots, c0:] = li.to_bf16_bits(rows * f[:, None])
        else:
            rows = li.bf16_bits_to_f32(x["k_cache"][pages, slots])
            x["k_cache"][pages, slots] = li.to_bf16_bits(rows * f[:, None, None])


@pytest.mark.parametrize("kind,h_q,splits,direction", [
    ("mla", 128, 0, "rise"), ("mla", 128, 5, "rise"), ("mla", 128, 0, "fall"),
    ("mla", 16, 0, "rise"), ("mla", 16, 3, "fall"), ("gqa", 32, 0, "rise"), ("gqa", 32, 4, "fall")])
def test_running_maximum_moves_along_the_cache(lkv, oracle, kind, h_q, splits, direction):
    """Scores whose spread grows (or shrinks) many times over along each
    sequence, so that the lazy reference maximum moves several times in the middle of a
    share (rising) or is set early and later tiles are small (falling), with
    random values: the output and LSE must still meet the oracle, which
    catches a wrong rescale factor (not only a missing one)."""
    seqlens = (700, 1500, 64)
    if kind == "mla":
        w, x = small_mla(1400 + h_q + splits + (1 if direction == "fall" else 0), h_q=h_q,
                         seqlens=seqlens)
    else:
        w, x = _gqa_small(1450 + splits + (1 if direction == "fall" else 0), h_q=h_q, n_kv=8,
                          seqlens=seqlens)
    _scale_keys_along_sequence(x, w, kind, direction)
    note(f"case running maximum {kind} h_q={h_q} splits={splits} {direction}")
    if kind == "mla":
        out, lse = run_mla(lkv, w, mla_device_inputs(x, w, torch), x=x, num_splits=splits)
        ro, rl = oracle_mla(oracle, w, x)
    else:
        out, lse = _run_gqa(lkv, w, x, num_splits=splits)
        ro, rl = _oracle_gqa(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl,
                 what=f"running maximum {kind} h_q={h_q} splits={splits} {direction}")


# ---------------------------------------------------- LKV_DEBUG_CHECKS=1
_DEBUG_CHILD = r"""
import math, sys
import torch
import latent_kv_decode_amd as lkv
import lkv_inputs as li
from tests.gpu_common import mla_device_inputs, run_mla
lkv.load_library()
w = li.Workload(name="dbg", kind="mla", dtype="bf16", B=3, h_q=128, s_q=1, page_size=64, n_lat=1,
                d_c=512, d_rope=64, seqlens=(100, 300, 65), table="shuffled", causal=True,
                max_pages=None, scale=1 / math.sqrt(576), seed=31)
x = li.generate(w)
d = mla_device_inputs(x, w, torch)
npg = int(x["num_pages"])
run_mla(lkv, w, d, num_pages=npg)
torch.cuda.synchronize()
print("good call ok", flush=True)
# every page of the pool is used, so a pool one page smaller leaves one
# table entry outside it (that page exists in memory)
try:
    run_mla(lkv, w, d, num_pages=npg - 1)
    print("bad page accepted", flush=True)
except lkv.LkvError as e:
    print("bad page rejected", e.status, flush=True)
# a length past max_pages * page_size in the first sequence (the row after
# it in the table holds valid pages)
sl = d["seqlens"].clone()
sl[0] = x["block_table"].shape[1] * w.page_size + 1
try:
    run_mla(lkv, w, dict(d, seqlens=sl), num_pages=npg)
    print("bad length accepted", flush=True)
except lkv.LkvError as e:
    print("bad length rejected", e.status, flush=True)
"""


def test_debug_checks_read_back_the_device_contract():
    """LKV_DEBUG_CHECKS=1 (read once per process, so the calls run in a child
    process): with no host copies given, the library reads the lengths and
    the block table back from the device and rejects a table entry outside
    the pool and a length past max_pages * page_size before any launch
    (LKV_ERR_SHAPE = 2); a valid call still runs."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, LKV_DEBUG_CHECKS="1", PYTHONPATH=root)
    note("case LKV_DEBUG_CHECKS=1 child process")
    r = subprocess.run([sys.executable, "-c", _DEBUG_CHILD], env=env, cwd=root, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert "good call ok" in lines, r.stdout
    assert "bad page rejected 2" in lines, r.stdout
    assert "bad length rejected 2" in lines, r.stdout


# ------------------------------------------------------------------ limits
def test_mla_max_query_tokens(lkv, oracle):
    """s_q = 64, the largest the ABI takes: 1024 query rows on one latent head
    (16 row tiles on the many-row kernel), one sequence shorter than s_q so
    that its first rows see nothing under causal masking."""
    w, x = small_mla(1200, h_q=16, s_q=64, seqlens=(40, 300))
    note("case mla s_q=64 h_q=16")
    d = mla_device_inputs(x, w, torch)
    out, lse = run_mla(lkv, w, d, x=x)
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what="mla s_q=64")


def test_gqa_max_query_tokens(lkv, oracle):
    """s_q = 64 with one query head per KV head: 64 rows per KV head, two
    32-row tiles, causal masking inside the step."""
    w, x = _gqa_small(1201, h_q=8, n_kv=8, s_q=64, seqlens=(64, 200, 90))
    note("case gqa s_q=64 h_q=8 n_kv=8")
    out, lse = _run_gqa(lkv, w, x)
    ro, rl = _oracle_gqa(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what="gqa s_q=64")


@pytest.mark.parametrize("kind,page", [("mla", 1), ("mla", 1000), ("mla16", 1), ("gqa", 1),
                                       ("gqa", 1000)])
def test_extreme_page_sizes(lkv, oracle, kind, page):
    """One-token pages (every token its own block-table entry) and pages
    larger than any sequence, not a power of two."""
    note(f"case page_size={page} {kind}")
    if kind == "gqa":
        w, x = _gqa_small(1210 + page, h_q=32, n_kv=8, page=page, seqlens=(100, 333, 65))
        out, lse = _run_gqa(lkv, w, x)
        ro, rl = _oracle_gqa(oracle, w, x)
    else:
        w, x = small_mla(1220 + page, h_q=128 if kind == "mla" else 16, page=page,
                         seqlens=(100, 333, 65))
        out, lse = run_mla(lkv, w, mla_device_inputs(x, w, torch), x=x)
        ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"{kind} page={page}")


@pytest.mark.parametrize("h_q,splits", [(128, 0), (128, 7), (16, 0), (16, 7)])
def test_many_short_sequences(lkv, oracle, h_q, splits):
    """300 sequences of 1..40 tokens: many sequences per share, shares that
    start and end inside a sequence's only tile."""
    rng = np.random.default_rng(1230 + h_q)
    seqlens = tuple(int(v) for v in rng.integers(1, 41, size=300))
    w, x = small_mla(1231 + h_q + splits, h_q=h_q, seqlens=seqlens)
    note(f"case 300 short sequences h_q={h_q} splits={splits}")
    out, lse = run_mla(lkv, w, mla_device_inputs(x, w, torch), x=x, num_splits=splits)
    ro, rl = oracle_mla(oracle, w, x)
    assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"short h_q={h_q}")


@pytest.mark.parametrize("kind", ["gqa", "mla"])
def test_fp8_scale_not_a_power_of_two(lkv, oracle, kind):
    """An 8-bit cache whose scale is not a power of two (the folded scales
    round in float32; the oracle takes kv_scale * code in float64)."""
    from dataclasses import replace
    if kind == "gqa":
        w, _ = _gqa_small(1240, h_q=128, n_kv=8, d_rope=64, s_q=2, cache="fp8")
    else:
        w, _ = small_mla(1241, h_q=128, seqlens=(300, 65, 700), cache="fp8")
    w = replace(w, kv_scale=0.0371)
    x = li.generate(w)
    note(f"case fp8 kv_scale=0.0371 {kind}")
    if kind == "gqa":
        out, lse = _run_gqa(lkv, w, x, **_fp8(w))
        ro, rl = _oracle_gqa(oracle, w, dequantised(oracle, x, GQA_KEYS + ["k_rope"], ["q", "q_rope"]))
    else:
        out, lse = run_mla(lkv, w, mla_device_inputs(x, w, torch), x=x, **_fp8(w))
        ro, rl = oracle_mla(oracle, w, dequantised(oracle, x, ["kv"], ["q_nope", "q_rope"]))
    assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"fp8 scale {kind}")


# ------------------------------------------------------- full-size workloads
FULL = [("dsv3_mla_b64_l4096", 96), ("gla2_b128_l8192", 64), ("ragged_mla_b16_sq1", 48),
        ("ragged_mla_b16_sq2", 48), ("mtp_mla_b64_l4096_sq4", 64), ("gta_b128_l8192", 64)]


@pytest.mark.parametrize("name,nrows", FULL)
def test_full_size_mla_sampled(lkv, oracle, name, nrows):
    w = li.workload(name)
    note(f"case full {name}: generating inputs")
    x = li.generate(w)
    d = mla_device_inputs(x, w, torch)
    note(f"case full {name}: running GPU")
    out, lse = run_mla(lkv, w, d, x=x)
    torch.cuda.synchronize()
    rows = li.sample_rows(11, w.B, w.s_q, w.h_q, nrows)
    ro, rl = oracle_mla(oracle, w, x, rows=rows)
    got, gl = from_dev(out), from_dev(lse)
    assert np.isfinite(got).all() and np.isfinite(gl).all()
    assert_close(rows_of(got, rows), rows_of(ro, rows), rows_of(gl, rows), rows_of(rl, rows),
                 what=name)


@pytest.mark.parametrize("name", ["gqa_b128_l8192", "vha_gqa2_b64_l8192"])
def test_full_size_gqa_sampled(lkv, oracle, name):
    w = li.workload(name)
    note(f"case full {name}: generating inputs")
    x = li.generate(w)
    out, lse = _run_gqa(lkv, w, x)
    torch.cuda.synchronize()
    rows = li.sample_rows(12, w.B, w.s_q, w.h_q, 64)
    ro, rl = _oracle_gqa(oracle, w, x, rows=rows)
    got, gl = from_dev(out), from_dev(lse)
    assert np.isfinite(got).all()
    assert_close(rows_of(got, rows), rows_of(ro, rows), rows_of(gl, rows), rows_of(rl, rows),
                 what=f"{name} full")


@pytest.mark.parametrize("name,nrows", [("dsv3_mla_b64_l4096_fp8", 64),
                                        ("gla2_b128_l8192_fp8", 48), ("gqa_b128_l8192_fp8", 48)])
def test_full_size_fp8_sampled(lkv, oracle, name, nrows):
    w = li.workload(name)
    note(f"case full {name}: generating inputs")
    x = li.generate(w)
    note(f"case full {name}: running GPU")
    if w.kind == "gqa":
        out, lse = _run_gqa(lkv, w, x, **_fp8(w))
    else:
        out, lse = run_mla(lkv, w, mla_device_inputs(x, w, torch), x=x, **_fp8(w))
    torch.cuda.synchronize()
    rows = li.sample_rows(14, w.B, w.s_q, w.h_q, nrows)
    if w.kind == "gqa":
        ro, rl = _oracle_gqa(oracle, w, dequantised(oracle, x, GQA_KEYS, ["q"]), rows=rows)
    else:
        ro, rl = oracle_mla(oracle, w, dequantised(oracle, x, ["kv"], ["q_nope", "q_rope"]),
                            rows=rows)
    got, gl = from_dev(out), from_dev(lse)
    assert np.isfinite(got).all() and np.isfinite(gl).all()
    assert_close(rows_of(got, rows), rows_of(ro, rows), rows_of(gl, rows), rows_of(rl, rows),
                 what=name)


@pytest.mark.parametrize("name", ["gqla_grouped_b64_l4096_sq2", "gqla_g4_b64_l4096_sq1"])
def test_full_size_gqla_grouped_sampled(lkv, oracle, name):
    w = li.workload(name)
    note(f"case full {name}: generating inputs")
    x = li.generate(w)
    kv, k_out, v_out = _expand_gpu(lkv, w, x)
    flat = kv.reshape(-1)
    out, lse = lkv.lkv_gqa_decode(to_dev(x["q_nope_h"], torch), to_dev(x["q_rope"], torch), k_out,
                                  v_out, flat[w.d_c:], torch.from_numpy(x["block_table"]).cuda(),
                                  torch.from_numpy(x["seqlens"]).cuda(), n_kv=w.n_kv,
                                  page_size=w.page_size, softmax_scale=w.scale,
                                  rope_tok_stride=w.d_c + w.d_rope, seqlens_host=x["seqlens"])
    torch.cuda.synchronize()
    # oracle grouped path on rows sampled from eight sequences spread over the
    # batch (first and last included): fp64 expansion of just those
    # sequences' tokens (their pages copied into a compact pool), then O3 on
    # the sampled rows
    seqs = sorted(set(int(v) for v in np.linspace(0, w.B - 1, 8).round()))
    per = w.s_q * w.h_q
    rng = np.random.default_rng(13)
    rows = np.sort(np.concatenate([s * per + rng.choice(per, 8, replace=False) for s in seqs]))
    rows = rows.astype(np.int32)
    pages = [x["block_table"][s, : (int(x["seqlens"][s]) + 63) // 64] for s in seqs]
    sub_bt = np.full((len(seqs), x["block_table"].shape[1]), -1, np.int32)
    pool = []
    for i, pg in enumerate(pages):
        sub_bt[i, : len(pg)] = np.arange(len(pool), len(pool) + len(pg))
        pool.extend(pg.tolist())
    sub_kv = x["kv"][np.array(pool)]
    sub_sl = x["seqlens"][seqs]
    wuk, wuv = _w64(x, "w_uk"), _w64(x, "w_uv")
    rk, rv = oracle.expand_latent(sub_kv.reshape(-1), wuk, wuv, sub_bt, sub_sl,
                                  page_size=w.page_size, num_pages=len(pool),
                                  kv_tok_stride=w.d_c + w.d_rope)
    kr64 = li.bf16_bits_to_f32(sub_kv[..., w.d_c:]).astype(np.float64)
    q_h = li.bf16_bits_to_f32(x["q_nope_h"]).astype(np.float64)[seqs]
    q_r = li.bf16_bits_to_f32(x["q_rope"]).astype(np.float64)[seqs]
    sub_rows = np.array([seqs.index(int(r) // per) * per + int(r) % per for r in rows], np.int32)
    note(f"case full {name}: oracle")
    ro, rl = oracle.gqa_decode(q_h, np.nan_to_num(rk), np.nan_to_num(rv), sub_bt, sub_sl,
                               n_kv=w.n_kv, d_h=w.d_h, page_size=w.page_size, scale=w.scale,
                               q_rope=q_r, k_rope=np.nan_to_num(kr64), d_rope=w.d_rope,
                               rows=sub_rows)
    got, gl = from_dev(out), from_dev(lse)
    assert np.isfinite(got).all()
    assert_close(rows_of(got, rows), rows_of(ro, sub_rows), rows_of(gl, rows), rows_of(rl, sub_rows),
                 what=f"{name} full")
