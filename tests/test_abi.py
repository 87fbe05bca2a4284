"""C ABI contract tests that need no GPU: the library loads, exports every
function include/lkv.h declares, its argument structs match the Python
binding byte for byte, and host-checkable preconditions fail fast with the
documented status (no launch, no device access)."""
import ctypes
import os
import re
import subprocess

import pytest

import latent_kv_decode_amd as lkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lkv.h")


@pytest.fixture(scope="module")
def lib():
    return lkv.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lkv_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert set(names) == set(lkv.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"{n} missing from liblkv.so"


def test_abi_version(lib):
    assert lkv.lkv_abi_version() == 5


def _c_layout(struct, fields):
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"lkv.h\"\nint main(){\n"
    src += f'printf("%zu\\n", sizeof({struct}));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof({struct}, {f}));\n'
    src += "return 0;}\n"
    tmp = os.path.join(os.environ.get("TMPDIR", "/tmp"), f"lkv_layout_{struct}")
    with open(tmp + ".c", "w") as fh:
        fh.write(src)
    subprocess.check_call(["gcc", "-I", os.path.join(ROOT, "include"), tmp + ".c", "-o", tmp])
    vals = [int(v) for v in subprocess.check_output([tmp]).split()]
    return vals[0], vals[1:]


@pytest.mark.parametrize("py,c", [(lkv.MlaArgs, "lkv_mla_args"), (lkv.GqaArgs, "lkv_gqa_args"),
                                  (lkv.ExpandArgs, "lkv_expand_args"),
                                  (lkv.CombineArgs, "lkv_combine_args"),
                                  (lkv.ProjArgs, "lkv_proj_args"),
                                  (lkv.AppendArgs, "lkv_append_args")])
def test_struct_layouts_match_header(py, c):
    fields = [f for f, _ in py._fields_]
    size, offs = _c_layout(c, fields)
    assert ctypes.sizeof(py) == size
    for (f, _), off in zip(py._fields_, offs):
        assert getattr(py, f).offset == off, f


FAKE = 0x10000  # never dereferenced: every case below fails validation first


def _mla(**kw):
    a = lkv.MlaArgs()
    a.struct_size = ctypes.sizeof(lkv.MlaArgs)
    a.dtype = lkv.LKV_BF16
    a.batch, a.s_q, a.h_q, a.n_latent, a.d_c, a.d_rope = 2, 1, 128, 1, 512, 64
    a.page_size, a.max_pages = 64, 4
    a.softmax_scale = 0.04
    a.causal = 1
    for f in ("q_nope", "q_rope", "c_kv", "k_rope", "block_table", "seqlens", "out", "lse"):
        setattr(a, f, FAKE)
    a.workspace = FAKE
    a.kv_tok_stride = 576
    a.rope_tok_stride = 576
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _status(lib, a):
    return lib.lkv_mla_decode(ctypes.byref(a))


@pytest.mark.parametrize("change,expect", [
    (dict(struct_size=12), 7),
    (dict(dtype=5), 3),
    (dict(h_q=100, n_latent=3), 2),
    (dict(d_c=320), 3),
    (dict(d_rope=16), 3),
    (dict(s_q=0), 2),
    (dict(batch=-1), 2),
    (dict(page_size=0), 2),
    (dict(num_splits=-2), 2),
    (dict(q_nope=None), 1),
    (dict(seqlens=None), 1),
    (dict(k_rope=None), 1),
    (dict(out=FAKE + 2), 4),
    (dict(kv_tok_stride=580), 4),
    (dict(kv_tok_stride=256), 2),
    (dict(workspace=None), 5),
    (dict(workspace=FAKE + 16), 4),
    (dict(softmax_scale=0.0), 2),
    (dict(softmax_scale=-0.05), 2),
    (dict(softmax_scale=float("inf")), 2),
    (dict(softmax_scale=float("nan")), 2),
    # 8-bit cache
    (dict(kv_fp8=1, kv_scale=0.0), 2),
    (dict(kv_fp8=1, kv_scale=float("nan")), 2),
    (dict(kv_fp8=1, kv_scale=0.1, dtype=0), 3),
    (dict(kv_fp8=1, kv_scale=0.1, h_q=16, d_rope=0), 3),  # few heads, 512 + 0
    (dict(kv_fp8=1, kv_scale=0.1, kv_tok_stride=584, rope_tok_stride=584), 4),
])
def test_mla_validation(lib, change, expect):
    st = _status(lib, _mla(**change))
    assert st == expect, (st, lkv.lkv_last_error())
    assert lkv.lkv_last_error() != ""


def test_null_args(lib):
    assert lib.lkv_mla_decode(None) == 1
    assert lib.lkv_gqa_decode(None) == 1
    assert lib.lkv_gqla_expand_latent(None) == 1
    assert lib.lkv_split_combine(None) == 1


def test_batch_zero_is_ok_without_pointers(lib):
    a = _mla(batch=0, q_nope=None, c_kv=None, out=None)
    assert _status(lib, a) == 0


def _gqa(**kw):
    a = lkv.GqaArgs()
    a.struct_size = ctypes.sizeof(lkv.GqaArgs)
    a.dtype = lkv.LKV_BF16
    a.batch, a.s_q, a.h_q, a.n_kv, a.d_h, a.d_rope = 2, 1, 32, 8, 128, 0
    a.page_size, a.max_pages = 64, 4
    a.softmax_scale = 0.09
    for f in ("q", "k_cache", "v_cache", "block_table", "seqlens", "out", "workspace"):
        setattr(a, f, FAKE)
    a.k_tok_stride = a.v_tok_stride = 1024
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("change,expect", [
    (dict(h_q=30), 2), (dict(d_h=96), 3), (dict(v_cache=None), 1), (dict(q_rope=FAKE), 2),
    (dict(d_rope=64), 1), (dict(v_tok_stride=512), 2), (dict(k_tok_stride=1028), 4),
    (dict(softmax_scale=-1.0), 2)])
def test_gqa_validation(lib, change, expect):
    st = lib.lkv_gqa_decode(ctypes.byref(_gqa(**change)))
    assert st == expect, (st, lkv.lkv_last_error())


def _expand(**kw):
    a = lkv.ExpandArgs()
    a.struct_size = ctypes.sizeof(lkv.ExpandArgs)
    a.dtype = lkv.LKV_BF16
    a.batch, a.g, a.d_c, a.d_h, a.page_size, a.max_pages = 2, 8, 512, 128, 64, 4
    for f in ("c_kv", "w_uk", "w_uv", "block_table", "seqlens", "k_out", "v_out"):
        setattr(a, f, FAKE)
    a.kv_tok_stride, a.k_tok_stride, a.v_tok_stride = 576, 1024, 1024
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("change,expect", [
    (dict(dtype=0), 3), (dict(d_c=1024), 3), (dict(d_h=96), 3), (dict(w_uv=None), 1),
    (dict(k_out=FAKE + 8), 4), (dict(kv_tok_stride=500), 4), (dict(k_tok_stride=512), 2),
    (dict(g=0), 2), (dict(struct_size=3), 7),
    # 8-bit expanded caches
    (dict(out_fp8=1, out_scale=0.0), 2), (dict(out_fp8=1, out_scale=float("inf")), 2),
    (dict(out_fp8=1, out_scale=0.1, k_tok_stride=1028), 4)])
def test_expand_validation(lib, change, expect):
    st = lib.lkv_gqla_expand_latent(ctypes.byref(_expand(**change)))
    assert st == expect, (st, lkv.lkv_last_error())


def _combine(**kw):
    a = lkv.CombineArgs()
    a.struct_size = ctypes.sizeof(lkv.CombineArgs)
    a.dtype = lkv.LKV_BF16
    a.batch, a.s_q, a.h_q, a.d_v, a.n_work = 2, 1, 16, 512, 4
    for f in ("o_part", "lse_part", "work_offsets", "out"):
        setattr(a, f, FAKE)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("change,expect", [
    (dict(d_v=6), 3), (dict(d_v=2048), 3), (dict(o_part=None), 1), (dict(o_part=FAKE + 4), 4),
    (dict(dtype=9), 3), (dict(s_q=0), 2)])
def test_combine_validation(lib, change, expect):
    st = lib.lkv_split_combine(ctypes.byref(_combine(**change)))
    assert st == expect, (st, lkv.lkv_last_error())


def _proj(**kw):
    a = lkv.ProjArgs()
    a.struct_size = ctypes.sizeof(lkv.ProjArgs)
    a.dtype = lkv.LKV_BF16
    a.batch, a.s_q, a.h_q, a.n_w, a.d_c, a.d_h = 2, 1, 128, 8, 512, 128
    a.x = a.w = a.y = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("fn", ["lkv_absorb_query", "lkv_up_project"])
@pytest.mark.parametrize("change,expect", [
    (dict(struct_size=8), 7), (dict(dtype=0), 3), (dict(h_q=100), 2), (dict(n_w=0), 2),
    (dict(d_c=96), 3), (dict(d_h=32), 3), (dict(x=None), 1), (dict(y=FAKE + 8), 4),
    (dict(s_q=0), 2)])
def test_proj_validation(lib, fn, change, expect):
    st = getattr(lib, fn)(ctypes.byref(_proj(**change)))
    assert st == expect, (st, lkv.lkv_last_error())


def _append(**kw):
    a = lkv.AppendArgs()
    a.struct_size = ctypes.sizeof(lkv.AppendArgs)
    a.dtype = lkv.LKV_BF16
    a.batch, a.s_q, a.width, a.page_size, a.max_pages = 2, 1, 576, 64, 4
    a.src = a.cache = a.block_table = a.seqlens = FAKE
    a.tok_stride = 576
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("change,expect", [
    (dict(struct_size=8), 7), (dict(dtype=4), 3), (dict(width=0), 2), (dict(width=580, tok_stride=1168), 4),
    (dict(tok_stride=500), 2), (dict(tok_stride=580), 4), (dict(cache=FAKE + 2), 4),
    (dict(seqlens=None), 1), (dict(page_size=0), 2),
    # 8-bit cache: bf16 source only, a usable scale, 16-byte rows of codes
    (dict(out_fp8=1, out_scale=1.0, dtype=lkv.LKV_F32), 3), (dict(out_fp8=1, out_scale=0.0), 2),
    (dict(out_fp8=1, out_scale=-1.0), 2), (dict(out_fp8=1, out_scale=float("nan")), 2),
    (dict(out_fp8=1, out_scale=float("inf")), 2), (dict(out_fp8=1, out_scale=1e-39), 2),
    (dict(out_fp8=1, out_scale=1.0, width=584, tok_stride=584), 4),
    (dict(out_fp8=1, out_scale=1.0, tok_stride=580), 4),
    (dict(out_fp8=1, out_scale=1.0, width=32, tok_stride=48, batch=0), 0)])
def test_append_validation(lib, change, expect):
    st = lib.lkv_append_tokens(ctypes.byref(_append(**change)))
    assert st == expect, (st, lkv.lkv_last_error())


def test_proj_and_append_batch_zero_ok(lib):
    assert lib.lkv_absorb_query(ctypes.byref(_proj(batch=0, x=None, w=None, y=None))) == 1
    assert lib.lkv_absorb_query(ctypes.byref(_proj(batch=0))) == 0
    assert lib.lkv_append_tokens(ctypes.byref(_append(batch=0))) == 0


def test_binding_version_matches_header():
    hdr = open(os.path.join(ROOT, "include", "lkv.h")).read()
    m = re.search(r"#define LKV_ABI_VERSION (\d+)", hdr)
    assert m and int(m.group(1)) == lkv.ABI_VERSION


def test_binding_raises_when_library_missing(tmp_path):
    with pytest.raises(ImportError):
        lkv._lib_backup = lkv._lib
        try:
            lkv._lib = None
            lkv.load_library(str(tmp_path / "nope.so"))
        finally:
            lkv._lib = lkv._lib_backup


# ------------------------------------------- host-side contract checks
def _host(arr):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


# max_pages 4, page_size 64: lengths up to 256; a pool of 6 pages
TABLE_OK = [[3, 0, -1, -1], [5, 1, 2, 4]]


@pytest.mark.parametrize("seqlens,table,num_pages,bad", [
    ([100, 256], TABLE_OK, 6, None),           # padding past the used pages is never read
    ([100, 256], None, 0, None),               # lengths only
    ([100, 257], None, 0, "seqlens[1]"),       # longer than max_pages * page_size
    ([-1, 10], None, 0, "seqlens[0]"),
    ([129, 10], TABLE_OK, 6, "block_table[0][2]"),   # a used page with id -1
    ([100, 256], TABLE_OK, 5, "block_table[1][0]"),  # id 5 outside a pool of 5 pages
    ([100, 256], [[3, 0, -1, -1], [5, 1, -7, 4]], 0, "block_table[1][2]"),
    ([0, 0], [[-1] * 4, [-1] * 4], 6, None),   # empty sequences use no page
])
@pytest.mark.parametrize("entry", ["mla", "gqa", "expand", "append"])
def test_host_contract_checks(lib, entry, seqlens, table, num_pages, bad):
    """With host copies of the lengths (and the block table), every length
    must lie in [0, max_pages * page_size] and every entry of a used page must
    name a page of the pool; a violation is LKV_ERR_SHAPE before any launch.
    Inputs that pass go on to the launch (LKV_ERR_HIP without a GPU)."""
    sl, sl_p = _host(seqlens)
    bt, bt_p = _host(table) if table is not None else (None, None)
    a, fn = {"mla": (_mla, lib.lkv_mla_decode), "gqa": (_gqa, lib.lkv_gqa_decode),
             "expand": (_expand, lib.lkv_gqla_expand_latent),
             "append": (_append, lib.lkv_append_tokens)}[entry]
    args = a(seqlens_host=sl_p, block_table_host=bt_p, num_pages=num_pages)
    st = fn(ctypes.byref(args))
    if bad is None:
        assert st in (0, 6), (st, lkv.lkv_last_error())
    else:
        assert st == 2, (st, lkv.lkv_last_error())
        assert bad in lkv.lkv_last_error()


def test_expand_bf16_strides_multiple_of_8(lib):
    """The bf16 expanded cache leaves in 16-byte pieces: strides must be
    multiples of 8 elements."""
    assert lib.lkv_gqla_expand_latent(ctypes.byref(_expand(k_tok_stride=1028))) == 4
    assert lib.lkv_gqla_expand_latent(ctypes.byref(_expand(v_tok_stride=1036))) == 4
