#!/usr/bin/env python3
"""Benchmark: decode attention over a compressed KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one call of the decode path over one batch of synthetic inputs
already resident in HBM (for the latent path: the MLA absorbed decode kernel,
plus the split-KV combine when any sequence is split).  The default workload
is the DeepSeek-V3-shaped MLA absorbed decode: batch 64, 128 query heads over
a 512-wide latent plus a 64-wide shared RoPE key, 4096 cache tokens each,
64-token pages, shuffled block table, bf16 with fp32 accumulation.

Timing: W untimed warm-up steps, then K timed steps bracketed by device
synchronisation.  HIP events on the stream the library launches on time each
step (attention kernel + split-KV combine), and a second pair, recorded by the
library itself around the attention kernel (kernel_events), times that kernel
alone for the roofline.  Four independent copies of the cache rotate from step
to step so that the 256 MB Infinity Cache cannot hold the working set.

    python bench.py --calibrate-copy
runs only a plain device-to-device copy of a known size (for scaling the
FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 run to bytes).

Printed: one JSON line with throughput (tokens/s), the roofline of the
dominant kernel (algorithmic bytes per launch over its mean duration against
the 8 TB/s HBM peak), the MFMA rate against the 2.5 PFLOP/s bf16 peak, and
the fp64 CPU oracle timed on this host on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn tokens/s + HBM GB/s & MFMA TFLOP/s (% roofline), B=64 L=4096"
COUNTERS = os.path.join(ROOT, "profiles", "mla_decode_dsv3_b64_l4096_counters.json")
KERNEL_SRC = os.path.join(ROOT, "latent_kv_decode_amd", "csrc", "decode_wide.hip")
COPY_BYTES = 1 << 30
ROTATE = 4


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    if c.get("kernel_source_sha") != kernel_sha():
        return None
    return c.get("hbm_bytes_per_launch")


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime (ctypes): the library
    records them on its own launch stream around the attention kernel."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")

    def create(self):
        e = self.ct.c_void_p()
        assert self.hip.hipEventCreate(self.ct.byref(e)) == 0
        return e.value

    def elapsed_ms(self, e0, e1):
        ms = self.ct.c_float()
        assert self.hip.hipEventSynchronize(self.ct.c_void_p(e1)) == 0
        assert self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(e0), self.ct.c_void_p(e1)) == 0
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(self.ct.c_void_p(e))


def calibrate_copy(steps):
    """A plain 1 GiB device copy, `steps` times: FETCH_SIZE and WRITE_SIZE of
    this kernel in a rocprofv3 run give the counters' bytes-per-unit scale."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "steps": steps}), flush=True)


def to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cpu_baseline(w, x, budget_s: float):
    """The fp64 oracle, as it stands, on this host's cores: whole query
    tokens (all heads of a sequence) until about `budget_s` seconds of CPU
    work or the whole batch."""
    import oracle
    per_seq = w.s_q * w.h_q
    width = w.n_lat * w.d_c + w.d_rope
    kv = x["kv"].reshape(-1)
    done_seqs, elapsed = 0, 0.0
    chunk = 1
    while done_seqs < w.B and elapsed < budget_s:
        n = min(chunk, w.B - done_seqs)
        rows = np.arange(done_seqs * per_seq, (done_seqs + n) * per_seq, dtype=np.int32)
        t0 = time.perf_counter()
        oracle.mla_decode(x["q_nope"], x["q_rope"], kv, kv[w.n_lat * w.d_c:], x["block_table"],
                          x["seqlens"], n_lat=w.n_lat, d_c=w.d_c, d_rope=w.d_rope,
                          page_size=w.page_size, scale=w.scale, causal=w.causal,
                          kv_tok_stride=width, rope_tok_stride=width, rows=rows)
        elapsed += time.perf_counter() - t0
        done_seqs += n
        chunk = min(chunk * 2, 16)
    tokens = done_seqs * w.s_q
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done_seqs} of {w.B} sequences (all {w.h_q} heads, {w.s_q} query token(s) "
                      f"each, full cache length) of the timed workload; {elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3_mla_b64_l4096")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.steps if args.steps != 200 else 5)
        return

    import torch
    import latent_kv_decode_amd as lkv
    import lkv_inputs as li
    from latent_kv_decode_amd import roofline as rf

    lkv.load_library()
    w = li.workload(args.workload)
    if w.kind != "mla":
        print("bench.py times the latent (MLA / GLA) workloads", file=sys.stderr)
        sys.exit(2)
    log(f"[bench] generating {w.name}")
    x = li.generate(w)
    width = w.n_lat * w.d_c + w.d_rope
    kvs = [to_dev(x["kv"], torch).reshape(-1)]
    for _ in range(ROTATE - 1):
        kvs.append(kvs[0].clone())
    q_nope, q_rope = to_dev(x["q_nope"], torch), to_dev(x["q_rope"], torch)
    bt = torch.from_numpy(x["block_table"]).cuda()
    sl = torch.from_numpy(x["seqlens"]).cuda()
    out = torch.empty((w.B, w.s_q, w.h_q, w.d_c), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.s_q, w.h_q), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    hip = HipEvents()
    kev = [(hip.create(), hip.create()) for _ in range(args.steps)]

    def step(i, events=None):
        kv = kvs[i % ROTATE]
        lkv.lkv_mla_decode(q_nope, q_rope, kv, kv[w.n_lat * w.d_c:], bt, sl, n_latent=w.n_lat,
                           page_size=w.page_size, softmax_scale=w.scale, causal=w.causal,
                           kv_tok_stride=width, rope_tok_stride=width, num_splits=args.num_splits,
                           seqlens_host=x["seqlens"], out=out, lse=lse, stream=stream,
                           kernel_events=events)

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i, kev[i])
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]) * 1e-3  # seconds
    kern = np.array([hip.elapsed_ms(a, b) for a, b in kev]) * 1e-3
    for a, b in kev:
        hip.destroy(a)
        hip.destroy(b)
    t_step = float(per.mean())
    t_kern = float(kern.mean())
    ms_per_step = wall / args.steps * 1e3

    work = rf.mla_work(x["seqlens"], s_q=w.s_q, h_q=w.h_q, n_lat=w.n_lat, d_c=w.d_c,
                       d_rope=w.d_rope, page_size=w.page_size, causal=w.causal)
    tokens = w.B * w.s_q
    hbm = work.bytes / t_kern / 1e9
    tflops = work.flops / t_kern / 1e12

    # quick sampled parity check of the timed output against the oracle
    import oracle
    rows = li.sample_rows(5, w.B, w.s_q, w.h_q, 8)
    kv0 = x["kv"].reshape(-1)
    ro, _ = oracle.mla_decode(x["q_nope"], x["q_rope"], kv0, kv0[w.n_lat * w.d_c:],
                              x["block_table"], x["seqlens"], n_lat=w.n_lat, d_c=w.d_c,
                              d_rope=w.d_rope, page_size=w.page_size, scale=w.scale,
                              causal=w.causal, kv_tok_stride=width, rope_tok_stride=width,
                              rows=rows)
    got = out.float().cpu().numpy().reshape(-1, w.d_c)[rows]
    ref = ro.reshape(-1, w.d_c)[rows]
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))

    traffic = measured_traffic() if args.workload == "dsv3_mla_b64_l4096" else None
    result = {
        "metric": METRIC,
        "value": tokens / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "seq_len": int(x["seqlens"].max()),
                   "s_q": w.s_q, "h_q": w.h_q, "n_latent": w.n_lat, "d_c": w.d_c,
                   "d_rope": w.d_rope, "page_size": w.page_size, "table": w.table,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": hbm, "peak": rf.MI355X_HBM_GBPS, "unit": "GB/s",
                     "frac": hbm / rf.MI355X_HBM_GBPS, "traffic": traffic},
        "mfma": {"achieved": tflops, "peak": rf.MI355X_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / rf.MI355X_BF16_TFLOPS},
        "step_us": t_step * 1e6,
        "kernel_us": t_kern * 1e6,
        "kernel_us_p10_p90": [float(np.percentile(kern, 10) * 1e6), float(np.percentile(kern, 90) * 1e6)],
        "kernel": "mla_wide_kernel (attention); the step adds the split-KV combine",
        "algorithmic": {"bytes_per_launch": work.bytes, "flops_per_launch": work.flops,
                        "intensity": work.intensity},
        "parity_sample_rel_l2": rel,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (fp64 oracle)")
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
