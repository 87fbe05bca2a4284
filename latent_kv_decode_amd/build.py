"""Build liblkv.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m latent_kv_decode_amd.build

Every source under csrc/ is compiled to an object with hipcc for gfx950 and
the objects are linked into latent_kv_decode_amd/liblkv.so.  Packed fp32 VALU
instructions are disabled for device code (-packed-fp32-ops), as the kernels
rely on plain scalar fp32 arithmetic only.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblkv.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "decode_mfma.hip", "decode_split.hip", "decode_f32.hip", "combine.hip", "expand.hip",
           "proj.hip", "noalloc.hip"]

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# Host-code sanitizers for CPU tests of the boundary (liblkv_san.so): each
# -fsanitize= applies to the host pass only (-Xarch_host); device code is not
# instrumented.
SAN_OUT = os.path.join(HERE, "liblkv_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, extra=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


def build_sanitized(verbose: bool = False) -> str:
    """liblkv_san.so: the boundary's host code (abi.cpp: validation, planning,
    dispatch) built with AddressSanitizer and UndefinedBehaviorSanitizer, the
    kernel objects as in build().  It is loaded only by CPU tests, in a
    process that preloads the sanitizer runtime."""
    os.makedirs(BUILD, exist_ok=True)
    objs = [_compile("abi.cpp", SAN_FLAGS, "_san")]
    objs += [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    tmp = SAN_OUT + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, SAN_OUT)
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload)."""
    r = subprocess.run([HIPCC.replace("hipcc", "amdclang++"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = hits[0] if hits else ""
    return path


if __name__ == "__main__":
    build(verbose=True)
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        build_sanitized(verbose=True)
    sys.exit(0)
