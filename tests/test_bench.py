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


def test_timed_oracle_repeats_a_small_batch():
    """A batch that takes less than min_s is run again from its start (the
    tiny workload); a large batch stops at the budget or at its end."""
    import bench
    calls = []

    def run(s0, n):
        calls.append((s0, n))

    done, el = bench.timed_oracle(run, 2, budget_s=10.0, min_s=0.01)
    assert done >= 2 and all(0 <= s0 < 2 and s0 + n <= 2 for s0, n in calls)
    assert "run" in bench.seq_sample(done, 2) or done == 2
    calls.clear()
    done, _ = bench.timed_oracle(run, 64, budget_s=10.0, min_s=0.0)
    assert done == 64 and sum(n for _, n in calls) == 64
    assert bench.seq_sample(3, 64) == "3 of 64 sequences"


def test_oracle_thread_count_can_be_set():
    import oracle
    oracle.build(force=False)
    n = oracle.num_threads()
    oracle.set_num_threads(1)
    assert oracle.num_threads() == 1
    oracle.set_num_threads(n)
    assert oracle.num_threads() == n


def test_counter_fields_follow_the_kernel_source(tmp_path, monkeypatch):
    """MFMA busy and traffic come from a committed counter summary only while
    the kernel source it names is unchanged."""
    import json
    import bench
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    c = {"kernel_source": str(src), "kernel_source_sha": bench.source_sha(str(src)),
         "hbm_bytes_per_launch": 123.0,
         "busy": {"mfma_busy_frac": 0.25, "wait_any_frac": 0.5, "duration_ns": 9000.0}}
    (tmp_path / "w_counters.json").write_text(json.dumps(c))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", "/")
    f = bench.counter_fields("w")
    assert f["mfma_busy"] == 0.25 and f["wait_any"] == 0.5 and f["duration_us"] == 9.0
    assert bench.measured_traffic("w") == 123.0
    src.write_text("kernel v2")
    assert bench.counter_fields("w") is None and bench.measured_traffic("w") is None
    assert bench.counter_fields("absent") is None


def test_committed_counter_summaries_name_a_source():
    """Every committed counter summary names an existing kernel source and
    carries the busy figures."""
    import glob
    import json
    import bench
    files = glob.glob(os.path.join(ROOT, "profiles", "*_counters.json"))
    assert files
    for f in files:
        c = json.load(open(f))
        assert os.path.isfile(os.path.join(ROOT, c["kernel_source"])), f
        assert {"mfma_busy_frac", "wait_any_frac"} <= set(c["busy"]), f
