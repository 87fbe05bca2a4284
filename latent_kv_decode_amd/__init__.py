"""latent_kv_decode_amd -- decode attention over a compressed KV cache on
AMD Instinct MI355X (gfx950).

Thin Python binding of liblkv (include/lkv.h).  The functions here only
marshal torch tensors into the C argument structs and call the library; every
step of the decode path runs in the library's HIP kernels.  PyTorch supplies
device memory and the current stream.  If liblkv.so is missing the binding
raises: there is no fallback implementation.

Entry points (same names as the C ABI):
  lkv_mla_decode          MLA absorbed decode (and GLA with several latent heads)
  lkv_mla_decode_noalloc  the same with the library's static scratch (allocates nothing)
  lkv_gqa_decode          grouped-query decode over an expanded cache (GQLA GQA path, plain GQA)
  lkv_gqla_expand_latent  latent -> g key/value groups at cache-write time
  lkv_split_combine       LSE-weighted merge of split-KV partial results
  lkv_absorb_query        W_UK folded into the per-head query (before decode)
  lkv_up_project          W_UV applied to the latent output (after decode)
  lkv_append_tokens       cache write of a step's new tokens
plus lkv_mla_decode_workspace_size / lkv_gqa_decode_workspace_size,
lkv_abi_version and lkv_last_error.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LKV_LIBRARY names another build of the same library (the tests load a
# sanitizer build of the host code through it); default: the in-tree build
LIB_PATH = os.environ.get("LKV_LIBRARY") or os.path.join(_HERE, "liblkv.so")

LKV_OK = 0
LKV_F32, LKV_BF16 = 0, 1
STATUS_NAMES = {0: "LKV_OK", 1: "LKV_ERR_NULL", 2: "LKV_ERR_SHAPE", 3: "LKV_ERR_UNSUPPORTED",
                4: "LKV_ERR_ALIGN", 5: "LKV_ERR_WORKSPACE", 6: "LKV_ERR_HIP", 7: "LKV_ERR_STRUCT"}

EXPORTED = ["lkv_abi_version", "lkv_last_error", "lkv_mla_decode", "lkv_mla_decode_workspace_size",
            "lkv_mla_decode_noalloc", "lkv_gqa_decode", "lkv_gqa_decode_workspace_size",
            "lkv_gqla_expand_latent", "lkv_split_combine", "lkv_absorb_query", "lkv_up_project",
            "lkv_append_tokens"]

_V = ctypes.c_void_p
_I = ctypes.c_int32
_L = ctypes.c_int64


class MlaArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _I), ("batch", _I), ("s_q", _I),
                ("h_q", _I), ("n_latent", _I), ("d_c", _I), ("d_rope", _I), ("page_size", _I),
                ("max_pages", _I), ("softmax_scale", ctypes.c_float), ("causal", _I),
                ("num_splits", _I), ("q_nope", _V), ("q_rope", _V), ("c_kv", _V),
                ("kv_tok_stride", _L), ("k_rope", _V), ("rope_tok_stride", _L),
                ("block_table", _V), ("seqlens", _V), ("seqlens_host", _V), ("out", _V),
                ("lse", _V), ("workspace", _V), ("workspace_bytes", ctypes.c_size_t),
                ("stream", _V), ("kernel_events", _V * 2), ("kv_fp8", _I),
                ("kv_scale", ctypes.c_float), ("block_table_host", _V), ("num_pages", _L)]


class GqaArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _I), ("batch", _I), ("s_q", _I),
                ("h_q", _I), ("n_kv", _I), ("d_h", _I), ("d_rope", _I), ("page_size", _I),
                ("max_pages", _I), ("softmax_scale", ctypes.c_float), ("causal", _I),
                ("num_splits", _I), ("q", _V), ("q_rope", _V), ("k_cache", _V),
                ("k_tok_stride", _L), ("v_cache", _V), ("v_tok_stride", _L), ("k_rope", _V),
                ("rope_tok_stride", _L), ("block_table", _V), ("seqlens", _V),
                ("seqlens_host", _V), ("out", _V), ("lse", _V), ("workspace", _V),
                ("workspace_bytes", ctypes.c_size_t), ("stream", _V), ("kernel_events", _V * 2),
                ("kv_fp8", _I), ("kv_scale", ctypes.c_float), ("block_table_host", _V),
                ("num_pages", _L)]


class ExpandArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _I), ("batch", _I), ("g", _I),
                ("d_c", _I), ("d_h", _I), ("page_size", _I), ("max_pages", _I), ("c_kv", _V),
                ("kv_tok_stride", _L), ("w_uk", _V), ("w_uv", _V), ("block_table", _V),
                ("seqlens", _V), ("start_pos", _V), ("k_out", _V), ("k_tok_stride", _L),
                ("v_out", _V), ("v_tok_stride", _L), ("stream", _V), ("out_fp8", _I),
                ("out_scale", ctypes.c_float), ("seqlens_host", _V), ("block_table_host", _V),
                ("num_pages", _L)]


class CombineArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _I), ("batch", _I), ("s_q", _I),
                ("h_q", _I), ("d_v", _I), ("n_work", _I), ("o_part", _V), ("lse_part", _V),
                ("work_offsets", _V), ("out", _V), ("lse", _V), ("stream", _V)]


class ProjArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _I), ("batch", _I), ("s_q", _I),
                ("h_q", _I), ("n_w", _I), ("d_c", _I), ("d_h", _I), ("x", _V), ("w", _V),
                ("y", _V), ("stream", _V)]


class AppendArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", _I), ("batch", _I), ("s_q", _I),
                ("width", _I), ("page_size", _I), ("max_pages", _I), ("src", _V), ("cache", _V),
                ("tok_stride", _L), ("block_table", _V), ("seqlens", _V), ("stream", _V),
                ("seqlens_host", _V), ("block_table_host", _V), ("num_pages", _L),
                ("out_fp8", _I), ("out_scale", ctypes.c_float)]


class LkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


# LKV_ABI_VERSION of include/lkv.h that the argument structs below follow
ABI_VERSION = 5


def load_library(path: str = LIB_PATH):
    """Load liblkv.so (built by latent_kv_decode_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m latent_kv_decode_amd.build` "
                              "(the HIP library is the only implementation; there is no fallback)")
        lib = ctypes.CDLL(path)
        lib.lkv_abi_version.restype = ctypes.c_int
        lib.lkv_last_error.restype = ctypes.c_char_p
        if lib.lkv_abi_version() != ABI_VERSION:
            raise ImportError(f"{path} has ABI version {lib.lkv_abi_version()}, this binding's "
                              f"argument structs are version {ABI_VERSION}: rebuild the library")
        for name, argt in [("lkv_mla_decode", MlaArgs), ("lkv_mla_decode_noalloc", MlaArgs),
                           ("lkv_gqa_decode", GqaArgs),
                           ("lkv_gqla_expand_latent", ExpandArgs),
                           ("lkv_split_combine", CombineArgs),
                           ("lkv_absorb_query", ProjArgs), ("lkv_up_project", ProjArgs),
                           ("lkv_append_tokens", AppendArgs)]:
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(argt)]
        for name, argt in [("lkv_mla_decode_workspace_size", MlaArgs),
                           ("lkv_gqa_decode_workspace_size", GqaArgs)]:
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.POINTER(argt), ctypes.POINTER(ctypes.c_size_t)]
        _lib = lib
    return _lib


def lkv_abi_version() -> int:
    return int(load_library().lkv_abi_version())


def lkv_last_error() -> str:
    return load_library().lkv_last_error().decode()


def _check(status: int):
    if status != LKV_OK:
        raise LkvError(status, lkv_last_error())


# ----------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LKV_BF16
    if t.dtype == torch.float32:
        return LKV_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_obj(stream):
    return _torch().cuda.current_stream() if stream is None else stream


def _stream(stream):
    return ctypes.c_void_p(_stream_obj(stream).cuda_stream)


def _host_i32(x):
    """Host int32 array for seqlens_host / block_table_host (kept alive by the
    caller frame)."""
    import numpy as np
    if x is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


_workspaces: dict = {}


def _workspace(device, stream, nbytes: int):
    """Scratch buffer for calls that pass no workspace, one per (device,
    stream), grown on demand.  It is allocated with `stream` current, so
    torch's caching allocator hands its memory to another tensor only after
    the work queued on that stream (a buffer replaced when the size grows
    stays reserved for its stream's pending calls).  Under HIP graph capture
    the caller must pass the workspace: a graph keeps the pointer, and a
    cached buffer may be replaced later."""
    torch = _torch()
    if nbytes == 0:
        return None
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("pass workspace= explicitly when capturing a HIP graph (size from "
                           "lkv_*_decode_workspace_size); the cached default may be replaced later")
    key = (str(device), int(stream.cuda_stream))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream):
            ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


# ----------------------------------------------------------- entry points
def _set_events(a, kernel_events):
    if kernel_events is not None:
        e0, e1 = kernel_events
        a.kernel_events[0] = e0 or None
        a.kernel_events[1] = e1 or None


def _mla_args(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, n_latent, page_size,
              softmax_scale, causal, kv_tok_stride, rope_tok_stride, num_splits, kv_fp8=False,
              kv_scale=1.0):
    B, s_q, h_q, d_c = q_nope.shape
    d_rope = 0 if q_rope is None else q_rope.shape[-1]
    a = MlaArgs()
    a.struct_size = ctypes.sizeof(MlaArgs)
    a.dtype = _dtype_code(q_nope)
    a.batch, a.s_q, a.h_q, a.n_latent, a.d_c, a.d_rope = B, s_q, h_q, n_latent, d_c, d_rope
    a.page_size = page_size
    a.max_pages = block_table.shape[1]
    a.softmax_scale = float(softmax_scale)
    a.causal = int(bool(causal))
    a.num_splits = int(num_splits)
    a.q_nope, a.q_rope = _ptr(q_nope), _ptr(q_rope)
    a.c_kv, a.k_rope = _ptr(c_kv), _ptr(k_rope)
    a.kv_tok_stride = n_latent * d_c if kv_tok_stride is None else kv_tok_stride
    a.rope_tok_stride = d_rope if rope_tok_stride is None else rope_tok_stride
    a.block_table, a.seqlens = _ptr(block_table), _ptr(seqlens)
    a.kv_fp8, a.kv_scale = int(bool(kv_fp8)), float(kv_scale)
    return a


def lkv_mla_decode_workspace_size(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, *,
                                  n_latent=1, page_size, softmax_scale, causal=True,
                                  kv_tok_stride=None, rope_tok_stride=None, num_splits=0,
                                  kv_fp8=False, kv_scale=1.0) -> int:
    a = _mla_args(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, n_latent, page_size,
                  softmax_scale, causal, kv_tok_stride, rope_tok_stride, num_splits, kv_fp8,
                  kv_scale)
    n = ctypes.c_size_t(0)
    _check(load_library().lkv_mla_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return int(n.value)


def lkv_mla_decode(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, *, n_latent=1,
                   page_size, softmax_scale, causal=True, kv_tok_stride=None,
                   rope_tok_stride=None, num_splits=0, seqlens_host=None, out=None, lse=None,
                   return_lse=True, workspace=None, stream=None, kernel_events=None,
                   kv_fp8=False, kv_scale=1.0, block_table_host=None, num_pages=0):
    """MLA absorbed decode (lkv.h: lkv_mla_decode).  Returns (out, lse).

    q_nope [B, s_q, h_q, d_c], q_rope [B, s_q, h_q, d_rope] (or None with
    d_rope = 0); c_kv / k_rope are the paged caches (base pointers; element
    offsets follow kv_tok_stride / rope_tok_stride); block_table int32
    [B, max_pages]; seqlens int32 [B] on the device.  kernel_events: optional
    pair of raw hipEvent_t handles (ints) recorded around the attention kernel.
    kv_fp8 / kv_scale: the caches hold OCP E4M3 codes (torch.uint8) of the
    values kv_scale * code.  seqlens_host / block_table_host (host int32
    copies) and num_pages (cache pool size) turn on the library's host-side
    checks of lengths and table entries before the launch.
    """
    torch = _torch()
    a = _mla_args(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, n_latent, page_size,
                  softmax_scale, causal, kv_tok_stride, rope_tok_stride, num_splits, kv_fp8,
                  kv_scale)
    lib = load_library()
    B, s_q, h_q, d_c = q_nope.shape
    if out is None:
        out = torch.empty((B, s_q, h_q, d_c), dtype=q_nope.dtype, device=q_nope.device)
    if lse is None and return_lse:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q_nope.device)
    n = ctypes.c_size_t(0)
    _check(lib.lkv_mla_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    st = _stream_obj(stream)
    if workspace is None:
        workspace = _workspace(q_nope.device, st, n.value)
    sh, a.seqlens_host = _host_i32(seqlens_host)
    bh, a.block_table_host = _host_i32(block_table_host)
    a.num_pages = int(num_pages)
    a.out, a.lse = _ptr(out), _ptr(lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.stream = ctypes.c_void_p(st.cuda_stream)
    _set_events(a, kernel_events)
    _check(lib.lkv_mla_decode(ctypes.byref(a)))
    del sh, bh
    return out, lse


def lkv_mla_decode_noalloc(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, *, n_latent=1,
                           page_size, softmax_scale, causal=True, kv_tok_stride=None,
                           rope_tok_stride=None, num_splits=0, seqlens_host=None, out=None,
                           lse=None, return_lse=True, stream=None, kernel_events=None,
                           kv_fp8=False, kv_scale=1.0, block_table_host=None, num_pages=0):
    """lkv_mla_decode with the library's static device scratch in place of a
    workspace (lkv.h: lkv_mla_decode_noalloc): the library allocates nothing.
    Pass `out` (and `lse`) to keep the binding from allocating them.
    Returns (out, lse)."""
    torch = _torch()
    a = _mla_args(q_nope, q_rope, c_kv, k_rope, block_table, seqlens, n_latent, page_size,
                  softmax_scale, causal, kv_tok_stride, rope_tok_stride, num_splits, kv_fp8,
                  kv_scale)
    B, s_q, h_q, d_c = q_nope.shape
    if out is None:
        out = torch.empty((B, s_q, h_q, d_c), dtype=q_nope.dtype, device=q_nope.device)
    if lse is None and return_lse:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q_nope.device)
    sh, a.seqlens_host = _host_i32(seqlens_host)
    bh, a.block_table_host = _host_i32(block_table_host)
    a.num_pages = int(num_pages)
    a.out, a.lse = _ptr(out), _ptr(lse)
    a.stream = _stream(stream)
    _set_events(a, kernel_events)
    _check(load_library().lkv_mla_decode_noalloc(ctypes.byref(a)))
    del sh, bh
    return out, lse


def _gqa_args(q, q_rope, k_cache, v_cache, k_rope, block_table, seqlens, n_kv, page_size,
              softmax_scale, causal, k_tok_stride, v_tok_stride, rope_tok_stride, num_splits,
              kv_fp8=False, kv_scale=1.0):
    B, s_q, h_q, d_h = q.shape
    d_rope = 0 if q_rope is None else q_rope.shape[-1]
    a = GqaArgs()
    a.struct_size = ctypes.sizeof(GqaArgs)
    a.dtype = _dtype_code(q)
    a.batch, a.s_q, a.h_q, a.n_kv, a.d_h, a.d_rope = B, s_q, h_q, n_kv, d_h, d_rope
    a.page_size = page_size
    a.max_pages = block_table.shape[1]
    a.softmax_scale = float(softmax_scale)
    a.causal = int(bool(causal))
    a.num_splits = int(num_splits)
    a.q, a.q_rope = _ptr(q), _ptr(q_rope)
    a.k_cache, a.v_cache, a.k_rope = _ptr(k_cache), _ptr(v_cache), _ptr(k_rope)
    a.k_tok_stride = n_kv * d_h if k_tok_stride is None else k_tok_stride
    a.v_tok_stride = n_kv * d_h if v_tok_stride is None else v_tok_stride
    a.rope_tok_stride = d_rope if rope_tok_stride is None else rope_tok_stride
    a.block_table, a.seqlens = _ptr(block_table), _ptr(seqlens)
    a.kv_fp8, a.kv_scale = int(bool(kv_fp8)), float(kv_scale)
    return a


def lkv_gqa_decode_workspace_size(q, q_rope, k_cache, v_cache, k_rope, block_table, seqlens, *,
                                  n_kv, page_size, softmax_scale, causal=True, k_tok_stride=None,
                                  v_tok_stride=None, rope_tok_stride=None, num_splits=0,
                                  kv_fp8=False, kv_scale=1.0) -> int:
    a = _gqa_args(q, q_rope, k_cache, v_cache, k_rope, block_table, seqlens, n_kv, page_size,
                  softmax_scale, causal, k_tok_stride, v_tok_stride, rope_tok_stride, num_splits,
                  kv_fp8, kv_scale)
    n = ctypes.c_size_t(0)
    _check(load_library().lkv_gqa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    return int(n.value)


def lkv_gqa_decode(q, q_rope, k_cache, v_cache, k_rope, block_table, seqlens, *, n_kv, page_size,
                   softmax_scale, causal=True, k_tok_stride=None, v_tok_stride=None,
                   rope_tok_stride=None, num_splits=0, seqlens_host=None, out=None, lse=None,
                   return_lse=True, workspace=None, stream=None, kernel_events=None,
                   kv_fp8=False, kv_scale=1.0, block_table_host=None, num_pages=0):
    """Grouped-query decode over an expanded cache (lkv.h: lkv_gqa_decode).
    Returns (out [B, s_q, h_q, d_h], lse); kernel_events, kv_fp8, kv_scale
    and the host-side checks as in lkv_mla_decode."""
    torch = _torch()
    a = _gqa_args(q, q_rope, k_cache, v_cache, k_rope, block_table, seqlens, n_kv, page_size,
                  softmax_scale, causal, k_tok_stride, v_tok_stride, rope_tok_stride, num_splits,
                  kv_fp8, kv_scale)
    lib = load_library()
    B, s_q, h_q, d_h = q.shape
    if out is None:
        out = torch.empty((B, s_q, h_q, d_h), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q.device)
    n = ctypes.c_size_t(0)
    _check(lib.lkv_gqa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)))
    st = _stream_obj(stream)
    if workspace is None:
        workspace = _workspace(q.device, st, n.value)
    sh, a.seqlens_host = _host_i32(seqlens_host)
    bh, a.block_table_host = _host_i32(block_table_host)
    a.num_pages = int(num_pages)
    a.out, a.lse = _ptr(out), _ptr(lse)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.stream = ctypes.c_void_p(st.cuda_stream)
    _set_events(a, kernel_events)
    _check(lib.lkv_gqa_decode(ctypes.byref(a)))
    del sh, bh
    return out, lse


def lkv_gqla_expand_latent(c_kv, w_uk, w_uv, block_table, seqlens, k_out, v_out, *, page_size,
                           kv_tok_stride=None, k_tok_stride=None, v_tok_stride=None,
                           start_pos=None, stream=None, out_fp8=False, out_scale=1.0,
                           seqlens_host=None, block_table_host=None, num_pages=0):
    """Expand the latent into g key/value groups (lkv.h: lkv_gqla_expand_latent).
    w_uk, w_uv [g, d_c, d_h] bf16; k_out / v_out are written in place (bf16,
    or with out_fp8 torch.uint8 E4M3 codes of value / out_scale).  Host-side
    checks as in lkv_mla_decode."""
    g, d_c, d_h = w_uk.shape
    a = ExpandArgs()
    a.struct_size = ctypes.sizeof(ExpandArgs)
    a.dtype = _dtype_code(c_kv)
    a.batch = block_table.shape[0]
    a.g, a.d_c, a.d_h = g, d_c, d_h
    a.page_size = page_size
    a.max_pages = block_table.shape[1]
    a.c_kv = _ptr(c_kv)
    a.kv_tok_stride = d_c if kv_tok_stride is None else kv_tok_stride
    a.w_uk, a.w_uv = _ptr(w_uk), _ptr(w_uv)
    a.block_table, a.seqlens, a.start_pos = _ptr(block_table), _ptr(seqlens), _ptr(start_pos)
    a.k_out, a.v_out = _ptr(k_out), _ptr(v_out)
    a.k_tok_stride = g * d_h if k_tok_stride is None else k_tok_stride
    a.v_tok_stride = g * d_h if v_tok_stride is None else v_tok_stride
    a.stream = _stream(stream)
    a.out_fp8, a.out_scale = int(bool(out_fp8)), float(out_scale)
    sh, a.seqlens_host = _host_i32(seqlens_host)
    bh, a.block_table_host = _host_i32(block_table_host)
    a.num_pages = int(num_pages)
    _check(load_library().lkv_gqla_expand_latent(ctypes.byref(a)))
    del sh, bh
    return k_out, v_out


def lkv_split_combine(o_part, lse_part, work_offsets, *, out=None, lse=None, dtype=None,
                      return_lse=True, stream=None):
    """LSE-weighted merge of split-KV partials (lkv.h: lkv_split_combine).
    o_part float32 [n_work, s_q, h_q, d_v], lse_part [n_work, s_q, h_q],
    work_offsets int32 [B+1] (device).  Returns (out, lse)."""
    torch = _torch()
    n_work, s_q, h_q, d_v = o_part.shape
    B = work_offsets.shape[0] - 1
    dtype = dtype or (out.dtype if out is not None else torch.bfloat16)
    if out is None:
        out = torch.empty((B, s_q, h_q, d_v), dtype=dtype, device=o_part.device)
    if lse is None and return_lse:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=o_part.device)
    a = CombineArgs()
    a.struct_size = ctypes.sizeof(CombineArgs)
    a.dtype = _dtype_code(out)
    a.batch, a.s_q, a.h_q, a.d_v, a.n_work = B, s_q, h_q, d_v, n_work
    a.o_part, a.lse_part, a.work_offsets = _ptr(o_part), _ptr(lse_part), _ptr(work_offsets)
    a.out, a.lse = _ptr(out), _ptr(lse)
    a.stream = _stream(stream)
    _check(load_library().lkv_split_combine(ctypes.byref(a)))
    return out, lse


def _proj(name, x, w, out, stream, up):
    torch = _torch()
    B, s_q, h_q, k = x.shape
    n_w, d_c, d_h = w.shape
    if out is None:
        out = torch.empty((B, s_q, h_q, d_h if up else d_c), dtype=x.dtype, device=x.device)
    a = ProjArgs()
    a.struct_size = ctypes.sizeof(ProjArgs)
    a.dtype = _dtype_code(x)
    a.batch, a.s_q, a.h_q, a.n_w, a.d_c, a.d_h = B, s_q, h_q, n_w, d_c, d_h
    a.x, a.w, a.y = _ptr(x), _ptr(w), _ptr(out)
    a.stream = _stream(stream)
    _check(getattr(load_library(), name)(ctypes.byref(a)))
    return out


def lkv_absorb_query(q, w_uk, *, out=None, stream=None):
    """W_UK folded into the query (lkv.h: lkv_absorb_query): q [B, s_q, h_q,
    d_h], w_uk [n_w, d_c, d_h] -> [B, s_q, h_q, d_c]."""
    return _proj("lkv_absorb_query", q, w_uk, out, stream, up=False)


def lkv_up_project(o_latent, w_uv, *, out=None, stream=None):
    """W_UV applied to the latent output (lkv.h: lkv_up_project): o_latent
    [B, s_q, h_q, d_c], w_uv [n_w, d_c, d_h] -> [B, s_q, h_q, d_h]."""
    return _proj("lkv_up_project", o_latent, w_uv, out, stream, up=True)


def lkv_append_tokens(src, cache, block_table, seqlens, *, page_size, tok_stride=None,
                      stream=None, seqlens_host=None, block_table_host=None, num_pages=0,
                      out_fp8=False, out_scale=1.0):
    """Cache write of a step's new tokens (lkv.h: lkv_append_tokens): src
    [B, s_q, width] rows go to positions seqlens[b] - s_q + t of the paged
    cache (base pointer; row r at r * tok_stride elements).  With out_fp8 the
    cache (torch.uint8) takes E4M3 codes of the bf16 values / out_scale.
    Host-side checks as in lkv_mla_decode."""
    import torch
    B, s_q, width = src.shape
    want = torch.uint8 if out_fp8 else src.dtype
    if cache.dtype != want:
        raise ValueError(f"lkv_append_tokens: cache dtype {cache.dtype}, expected {want}")
    a = AppendArgs()
    a.struct_size = ctypes.sizeof(AppendArgs)
    a.dtype = _dtype_code(src)
    a.batch, a.s_q, a.width = B, s_q, width
    a.page_size, a.max_pages = page_size, block_table.shape[1]
    a.src, a.cache = _ptr(src), _ptr(cache)
    a.tok_stride = width if tok_stride is None else tok_stride
    a.block_table, a.seqlens = _ptr(block_table), _ptr(seqlens)
    a.stream = _stream(stream)
    sh, a.seqlens_host = _host_i32(seqlens_host)
    bh, a.block_table_host = _host_i32(block_table_host)
    a.num_pages = int(num_pages)
    a.out_fp8, a.out_scale = int(bool(out_fp8)), float(out_scale)
    _check(load_library().lkv_append_tokens(ctypes.byref(a)))
    del sh, bh
    return cache
