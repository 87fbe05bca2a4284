"""bench.py host logic (no GPU): the single-GPU contract and the oracle's
copy of an 8-bit workload."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_oracle_copy_of_an_8bit_workload():
    import bench
    import lkv_inputs as li
    import oracle
    oracle.build(force=False)
    w = li.workload("gqa_b128_l8192_fp8", B=2, seqlens=(70, 130))
    x = li.generate(w)
    y = bench.oracle_inputs(x, w, ["k_cache", "v_cache"], ["q"])
    assert y["k_cache"].dtype == np.float32 and y["q"].dtype == np.float32
    # the codes' values times the scale, through the oracle's decoding
    want = oracle.e4m3_to_f64(x["k_cache"], w.kv_scale)
    finite = np.isfinite(want)
    assert np.array_equal(y["k_cache"][finite], want[finite].astype(np.float32))
    assert np.array_equal(y["q"], li.bf16_bits_to_f32(x["q"]))
    # bf16 workloads pass through unchanged
    wb = li.workload("gqa_b128_l8192", B=2, seqlens=(70, 130))
    xb = li.generate(wb)
    assert bench.oracle_inputs(xb, wb, ["k_cache"], ["q"]) is xb
