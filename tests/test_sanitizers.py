"""The boundary's host code and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

liblkv_san.so is abi.cpp (validation, contract checks, planning, dispatch)
built with -fsanitize=address,undefined for the host pass, linked with the
regular kernel objects; the oracle is rebuilt with gcc's sanitizers.  Each
suite runs in a child process that preloads the matching sanitizer runtime
(Python itself is not instrumented) and must pass with no sanitizer report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _symbols(path):
    out = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True)
    return out.stdout


def _run_child(env_extra, test_file):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", test_file, "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-3000:]
    assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-3000:]
    return text


def test_boundary_host_code_under_sanitizers():
    from latent_kv_decode_amd import build as b
    lib = b.build_sanitized()
    syms = _symbols(lib)
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "abi.cpp is not instrumented"
    rt = b.sanitizer_runtime()
    if not rt:
        pytest.skip("no shared AddressSanitizer runtime found")
    text = _run_child({"LD_PRELOAD": rt, "LKV_LIBRARY": lib}, "tests/test_abi.py")
    assert " passed" in text


def test_oracle_under_sanitizers():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc has no shared AddressSanitizer runtime")
    env = {"LD_PRELOAD": asan, "LKV_ORACLE_SANITIZE": "1"}
    text = _run_child(env, "tests/test_oracle.py")
    assert " passed" in text
    lib = os.path.join(ROOT, "oracle", "liblkv_oracle_san.so")
    syms = _symbols(lib)
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "oracle.c is not instrumented"
