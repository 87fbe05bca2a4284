"""lkv_mla_decode_noalloc: the MLA decode entry point for callers that cannot
allocate, whose split partials live in the library's static device scratch.
Its output must equal lkv_mla_decode's (same kernels, same split plan) bit
for bit, on two calls in a row with the second input smaller than the first
(the scratch keeps the first call's contents), and both must meet the
oracle; arguments needing more scratch than the static array holds are
rejected before any launch."""
import numpy as np
import pytest

from tests.gpu_common import assert_close, from_dev, mla_device_inputs, note, oracle_mla, run_mla, \
    small_mla

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


def _noalloc(lkv, w, d, x, **kw):
    out = torch.full(d["q_nope"].shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(d["q_nope"].shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    return lkv.lkv_mla_decode_noalloc(d["q_nope"], d["q_rope"], d["c_kv"], d["k_rope"],
                                      d["block_table"], d["seqlens"], n_latent=w.n_lat,
                                      page_size=w.page_size, softmax_scale=w.scale,
                                      causal=w.causal, kv_tok_stride=d["kv_tok_stride"],
                                      rope_tok_stride=d["rope_tok_stride"],
                                      seqlens_host=x["seqlens"], out=out, lse=lse, **kw)


def test_noalloc_equals_workspace_entry_point(lkv, oracle):
    cases = [
        # 64 sequences of 128 heads: 128 shares, 48 MiB of partials (near the limit)
        dict(seed=2000, B=64, s_q=1, seqlens=[300 + 7 * i for i in range(64)], splits=0),
        # then a smaller input with several shares per sequence
        dict(seed=2001, B=3, s_q=2, seqlens=[700, 65, 2], splits=7),
    ]
    for c in cases:
        w, x = small_mla(c["seed"], B=c["B"], s_q=c["s_q"], seqlens=c["seqlens"])
        note(f"case noalloc B={c['B']} s_q={c['s_q']} splits={c['splits']}")
        d = mla_device_inputs(x, w, torch)
        ref_o, ref_l = run_mla(lkv, w, d, x=x, num_splits=c["splits"])
        out, lse = _noalloc(lkv, w, d, x, num_splits=c["splits"])
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
        assert torch.equal(lse, ref_l)
        ro, rl = oracle_mla(oracle, w, x)
        assert_close(from_dev(out), ro, from_dev(lse), rl, what=f"noalloc B={c['B']}")


def test_noalloc_rejects_more_than_the_static_scratch(lkv):
    """200 sequences of 128 heads need (200 + 128) x 128 x 512 float32
    partials, above the 64 MiB array: LKV_ERR_WORKSPACE, nothing launched
    (the output keeps its NaN fill)."""
    w, x = small_mla(2002, B=200, seqlens=[1] * 200)
    d = mla_device_inputs(x, w, torch)
    with pytest.raises(lkv.LkvError) as e:
        out, _ = _noalloc(lkv, w, d, x)
    assert e.value.status == 5 and "static" in str(e.value)
