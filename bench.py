#!/usr/bin/env python3
"""Benchmark: decode attention over a compressed KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one call of the decode path over one batch of synthetic inputs
already resident in HBM.  The default workload is the DeepSeek-V3-shaped MLA
absorbed decode: batch 64, 128 query heads over a 512-wide latent plus a
64-wide shared RoPE key, 4096 cache tokens each, 64-token pages, shuffled
block table, bf16 with fp32 accumulation (one step = the attention kernel plus
the split-KV combine).  Other workloads (lkv_inputs.WORKLOADS):
  gla2_b128_l8192, ragged_mla_b16_sq1, ragged_mla_b16_sq2   latent path
  gqa_b128_l8192                                             plain GQA
  gqla_grouped_b64_l4096_sq2   GQLA grouped path: the latent is expanded into
                               8 key/value groups once (timed separately, not
                               part of the step), then grouped decode
  dsv3_mla_b64_l4096_fp8, gla2_b128_l8192_fp8, gqa_b128_l8192_fp8
                               the same with 8-bit (OCP E4M3) caches

Timing: W untimed warm-up steps (default 150: the first ~100 steps of a run
are up to 20% slower while the chip settles), then K timed steps bracketed by
device synchronisation.  One pair of HIP events on the stream the library launches
on brackets the K steps (the step time is their span over K), and a pair on
every fourth step of the same timed region, attached by the library to the
attention kernel's own launch (kernel_events, no marker packets between
kernels), times that kernel alone for the roofline (a pair on every step adds
about 4 us to each step).  Four
independent copies of the cache rotate from step to step so that the 256 MB
Infinity Cache cannot hold the working set.

    python bench.py --calibrate-copy
runs only a plain device-to-device copy of a known size (for scaling the
FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 run to bytes).

Printed: one JSON line with throughput (tokens/s), the roofline of the
attention kernel (algorithmic bytes per launch over its mean duration against
the 8 TB/s HBM peak), the MFMA rate against the 2.5 PFLOP/s bf16 peak, and
the fp64 CPU oracle timed on this host on a bounded sample of the workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn tokens/s + HBM GB/s & MFMA TFLOP/s (% roofline), B=64 L=4096"
PROFILES = os.path.join(ROOT, "profiles")
ROTATE = 4
COPY_BYTES = 1 << 30


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_counters(workload: str):
    """The committed rocprofv3 counter summary of this workload's attention
    kernel (HBM bytes per launch, matrix-unit busy fraction, shader clock), or
    None when there is none or the kernel source changed since the counters
    were taken."""
    path = os.path.join(PROFILES, f"{workload}_counters.json")
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    src = os.path.join(ROOT, c.get("kernel_source", ""))
    if not os.path.isfile(src) or c.get("kernel_source_sha") != source_sha(src):
        return None
    return c


def counter_fields(workload: str):
    """The attention kernel's matrix-unit busy fraction (SQ_VALU_MFMA_BUSY_CYCLES
    over every SIMD's cycles at the published 2.4 GHz) and the fraction of
    wave time spent waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES), from the committed
    counter run of the same kernel source; None when there is none."""
    c = measured_counters(workload)
    if c is None or "busy" not in c:
        return None
    b = c["busy"]
    return {"mfma_busy": b["mfma_busy_frac"], "wait_any": b["wait_any_frac"],
            "duration_us": b["duration_ns"] / 1e3,
            "source": f"profiles/{workload}_counters.json (rocprofv3 --pmc)"}


def measured_traffic(workload: str):
    """HBM bytes per launch of the attention kernel (see measured_counters)."""
    c = measured_counters(workload)
    return None if c is None else c.get("hbm_bytes_per_launch")


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime (ctypes): the library
    attaches them to the attention kernel's launch on its own stream."""

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
        assert self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(e0),
                                            self.ct.c_void_p(e1)) == 0
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(self.ct.c_void_p(e))


def ramp(workload: str, n: int):
    """Per-step times from a cold start, an event pair around every step: first
    a plain device copy as large as the workload's cache (four rotating
    buffers), then the decode step itself.  Prints one JSON line with the
    medians of each block of 25 steps, which shows whether a slow start
    belongs to the chip (the copy slows too) or to the decode kernel."""
    import torch
    import latent_kv_decode_amd as lkv
    import lkv_inputs as li
    from latent_kv_decode_amd import roofline as rf
    lkv.load_library()
    stream = torch.cuda.current_stream()

    def series(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        return [round(float(np.median(us[i:i + 25])), 1) for i in range(0, n, 25)]

    w = li.workload(workload)
    x = li.generate(w)
    nbytes = sum(int(v.nbytes) for k, v in x.items() if k in ("kv", "k_cache", "v_cache"))
    src = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(4)]
    dst = [torch.empty_like(t) for t in src]
    for t in src:
        t.fill_(1)
    torch.cuda.synchronize()
    time.sleep(2.0)
    log(f"[bench] ramp: copy of {nbytes} bytes, {n} steps")
    cp = series(lambda i: dst[i % 4].copy_(src[i % 4]))
    del src, dst

    class Opt:
        num_splits = 0

    s = SETUPS[w.kind](w, x, Opt, torch, lkv, rf)
    torch.cuda.synchronize()
    time.sleep(2.0)
    log(f"[bench] ramp: {w.name} step, {n} steps")
    st = series(lambda i: s["step"](i))
    print(json.dumps({"ramp": w.name, "steps": n, "block": 25, "copy_bytes": nbytes,
                      "copy_us_median_per_block": cp, "step_us_median_per_block": st}), flush=True)


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


def f64(bits):
    import lkv_inputs as li
    return li.bf16_bits_to_f32(bits).astype(np.float64)


def timed_oracle(run_seqs, B: int, budget_s: float, min_s: float = 1.0):
    """Call run_seqs(s0, n) on growing groups of whole sequences until about
    budget_s seconds of oracle time or the whole batch; a batch that takes
    less than min_s is run again from its start until min_s has passed (the
    tiny workload).  Returns (sequences done, seconds)."""
    done, elapsed, chunk = 0, 0.0, 1
    while elapsed < budget_s and (done < B or elapsed < min_s):
        s0 = done % B
        n = min(chunk, B - s0)
        t0 = time.perf_counter()
        run_seqs(s0, n)
        elapsed += time.perf_counter() - t0
        done += n
        chunk = min(chunk * 2, 16)
    return done, elapsed


def seq_sample(done: int, B: int) -> str:
    """Words for the sequences one timed oracle sample covered."""
    if done <= B:
        return f"{done} of {B} sequences"
    return f"{done} sequence evaluations (the batch of {B} run {done / B:.0f} times)"


def oracle_inputs(x, w, keys, qkeys):
    """The oracle's copies of the inputs: an 8-bit cache dequantised to
    float32 (exact: E4M3 values times a power-of-two scale) through the
    oracle's own E4M3 decoding of all 256 codes, the queries widened to match;
    other workloads pass through.  Computed once."""
    if w.cache != "fp8":
        return x
    if "_oracle_copy" not in x:
        import oracle
        import lkv_inputs as li
        lut = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8), x["kv_scale"]).astype(np.float32)
        y = {k: lut[x[k]] for k in keys}
        y.update({k: li.bf16_bits_to_f32(x[k]) for k in qkeys})
        x["_oracle_copy"] = y
    return {**x, **x["_oracle_copy"]}


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


# ----------------------------------------------------------------- workloads
def setup_mla(w, x, args, torch, lkv, rf):
    import oracle
    import lkv_inputs as li
    width = w.n_lat * w.d_c + w.d_rope
    kvs = [to_dev(x["kv"], torch).reshape(-1)]
    for _ in range(ROTATE - 1):
        kvs.append(kvs[0].clone())
    q_nope, q_rope = to_dev(x["q_nope"], torch), to_dev(x["q_rope"], torch)
    bt = torch.from_numpy(x["block_table"]).cuda()
    sl = torch.from_numpy(x["seqlens"]).cuda()
    f32 = w.dtype == "f32"
    out = torch.empty((w.B, w.s_q, w.h_q, w.d_c), dtype=torch.float32 if f32 else torch.bfloat16,
                      device="cuda")
    lse = torch.empty((w.B, w.s_q, w.h_q), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fp8 = w.cache == "fp8"
    q8 = dict(kv_fp8=True, kv_scale=w.kv_scale) if fp8 else {}

    def step(i, events=None):
        kv = kvs[i % ROTATE]
        lkv.lkv_mla_decode(q_nope, q_rope, kv, kv[w.n_lat * w.d_c:], bt, sl, n_latent=w.n_lat,
                           page_size=w.page_size, softmax_scale=w.scale, causal=w.causal,
                           kv_tok_stride=width, rope_tok_stride=width, num_splits=args.num_splits,
                           seqlens_host=x["seqlens"], out=out, lse=lse, stream=stream,
                           kernel_events=events, **q8)

    def oracle_rows(rows):
        y = oracle_inputs(x, w, ["kv"], ["q_nope", "q_rope"])
        kv0 = y["kv"].reshape(-1)
        return oracle.mla_decode(y["q_nope"], y["q_rope"], kv0, kv0[w.n_lat * w.d_c:],
                                 x["block_table"], x["seqlens"], n_lat=w.n_lat, d_c=w.d_c,
                                 d_rope=w.d_rope, page_size=w.page_size, scale=w.scale,
                                 causal=w.causal, kv_tok_stride=width, rope_tok_stride=width,
                                 rows=rows)

    def parity():
        rows = li.sample_rows(5, w.B, w.s_q, w.h_q, 8)
        ro, _ = oracle_rows(rows)
        got = out.float().cpu().numpy().reshape(-1, w.d_c)[rows]
        return rel_l2(got, ro.reshape(-1, w.d_c)[rows])

    def cpu(budget):
        per = w.s_q * w.h_q
        done, el = timed_oracle(
            lambda s0, n: oracle_rows(np.arange(s0 * per, (s0 + n) * per, dtype=np.int32)),
            w.B, budget)
        return done, el, f"{seq_sample(done, w.B)} (all {w.h_q} heads, {w.s_q} query token(s) " \
                         f"each, full cache length) of the timed workload"

    work = rf.mla_work(x["seqlens"], s_q=w.s_q, h_q=w.h_q, n_lat=w.n_lat, d_c=w.d_c,
                       d_rope=w.d_rope, page_size=w.page_size, causal=w.causal,
                       cache_elem=1 if fp8 else (4 if f32 else 2), elem=4 if f32 else 2)
    many_rows = w.h_q // w.n_lat * w.s_q > 32 and w.d_c in (256, 512)
    kernel = "f32_decode_kernel" if f32 else "mla_split_kernel" if many_rows else "mfma_decode_kernel"
    return dict(step=step, work=work, parity=parity, cpu=cpu, out=out, kernel=kernel,
                config={"n_latent": w.n_lat, "d_c": w.d_c, "d_rope": w.d_rope,
                        "cache": "e4m3" if fp8 else "bf16"})


def setup_gqa(w, x, args, torch, lkv, rf):
    import oracle
    import lkv_inputs as li
    ks = [to_dev(x["k_cache"], torch)]
    vs = [to_dev(x["v_cache"], torch)]
    for _ in range(ROTATE - 1):
        ks.append(ks[0].clone())
        vs.append(vs[0].clone())
    q = to_dev(x["q"], torch)
    bt = torch.from_numpy(x["block_table"]).cuda()
    sl = torch.from_numpy(x["seqlens"]).cuda()
    out = torch.empty((w.B, w.s_q, w.h_q, w.d_h), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.s_q, w.h_q), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fp8 = w.cache == "fp8"
    q8 = dict(kv_fp8=True, kv_scale=w.kv_scale) if fp8 else {}

    def step(i, events=None):
        lkv.lkv_gqa_decode(q, None, ks[i % ROTATE], vs[i % ROTATE], None, bt, sl, n_kv=w.n_kv,
                           page_size=w.page_size, softmax_scale=w.scale, causal=w.causal,
                           num_splits=args.num_splits, seqlens_host=x["seqlens"], out=out,
                           lse=lse, stream=stream, kernel_events=events, **q8)

    def oracle_rows(rows):
        y = oracle_inputs(x, w, ["k_cache", "v_cache"], ["q"])
        return oracle.gqa_decode(y["q"], y["k_cache"], y["v_cache"], x["block_table"],
                                 x["seqlens"], n_kv=w.n_kv, d_h=w.d_h, page_size=w.page_size,
                                 scale=w.scale, causal=w.causal, rows=rows)

    def parity():
        rows = li.sample_rows(5, w.B, w.s_q, w.h_q, 8)
        ro, _ = oracle_rows(rows)
        got = out.float().cpu().numpy().reshape(-1, w.d_h)[rows]
        return rel_l2(got, ro.reshape(-1, w.d_h)[rows])

    def cpu(budget):
        per = w.s_q * w.h_q
        done, el = timed_oracle(
            lambda s0, n: oracle_rows(np.arange(s0 * per, (s0 + n) * per, dtype=np.int32)),
            w.B, budget)
        return done, el, f"{seq_sample(done, w.B)} (all {w.h_q} heads) of the timed workload"

    work = rf.gqa_work(x["seqlens"], s_q=w.s_q, h_q=w.h_q, n_kv=w.n_kv, d_h=w.d_h, d_rope=0,
                       page_size=w.page_size, causal=w.causal, cache_elem=1 if fp8 else 2)
    return dict(step=step, work=work, parity=parity, cpu=cpu, out=out, kernel="mfma_decode_kernel",
                config={"n_kv": w.n_kv, "d_h": w.d_h, "d_rope": 0,
                        "cache": "e4m3" if fp8 else "bf16"})


def setup_gqla(w, x, args, torch, lkv, rf):
    """GQLA grouped path: expand the latent once (timed on its own), then
    grouped decode over the expanded K/V plus the latent cache's RoPE part."""
    import oracle
    width = w.d_c + w.d_rope
    kv = to_dev(x["kv"], torch)
    num_pages, P = kv.shape[0], kv.shape[1]
    flat = kv.reshape(-1)
    wuk, wuv = to_dev(x["w_uk"], torch), to_dev(x["w_uv"], torch)
    bt = torch.from_numpy(x["block_table"]).cuda()
    sl = torch.from_numpy(x["seqlens"]).cuda()
    k0 = torch.empty((num_pages, P, w.n_kv, w.d_h), dtype=torch.bfloat16, device="cuda")
    v0 = torch.empty_like(k0)
    stream = torch.cuda.current_stream()

    def expand(k_out, v_out):
        lkv.lkv_gqla_expand_latent(flat, wuk, wuv, bt, sl, k_out, v_out, page_size=w.page_size,
                                   kv_tok_stride=width, stream=stream)

    for _ in range(2):
        expand(k0, v0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_exp = 5
    e0.record(stream)
    for _ in range(n_exp):
        expand(k0, v0)
    e1.record(stream)
    torch.cuda.synchronize()
    t_exp = e0.elapsed_time(e1) * 1e-3 / n_exp
    # the same expansion into 8-bit (E4M3) caches, scale 1/16
    k8 = torch.empty((num_pages, P, w.n_kv, w.d_h), dtype=torch.uint8, device="cuda")
    v8 = torch.empty_like(k8)

    def expand8():
        lkv.lkv_gqla_expand_latent(flat, wuk, wuv, bt, sl, k8, v8, page_size=w.page_size,
                                   kv_tok_stride=width, stream=stream, out_fp8=True,
                                   out_scale=1.0 / 16)

    for _ in range(2):
        expand8()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n_exp):
        expand8()
    e1.record(stream)
    torch.cuda.synchronize()
    t_exp8 = e0.elapsed_time(e1) * 1e-3 / n_exp
    del k8, v8
    # context for the expansion (not part of the path): the vendor library's
    # GEMM (torch.matmul, hipBLASLt) on the same product with contiguous
    # operands -- no gather through the block table, one output matrix --
    # timed the same way
    n_ctx = int(np.sum(x["seqlens"]))
    gen = torch.Generator(device="cuda").manual_seed(7)
    a_ctx = torch.randn((n_ctx, w.d_c), device="cuda", generator=gen).to(torch.bfloat16)
    w_ctx = torch.randn((2 * w.n_kv * w.d_h, w.d_c), device="cuda", generator=gen).to(torch.bfloat16)
    o_ctx = torch.empty((n_ctx, 2 * w.n_kv * w.d_h), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        torch.matmul(a_ctx, w_ctx.t(), out=o_ctx)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n_exp):
        torch.matmul(a_ctx, w_ctx.t(), out=o_ctx)
    e1.record(stream)
    torch.cuda.synchronize()
    t_gemm = e0.elapsed_time(e1) * 1e-3 / n_exp
    del a_ctx, w_ctx, o_ctx
    ks, vs = [k0], [v0]
    for _ in range(ROTATE - 1):
        ks.append(k0.clone())
        vs.append(v0.clone())
    q, q_rope = to_dev(x["q_nope_h"], torch), to_dev(x["q_rope"], torch)
    out = torch.empty((w.B, w.s_q, w.h_q, w.d_h), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.s_q, w.h_q), dtype=torch.float32, device="cuda")

    def step(i, events=None):
        lkv.lkv_gqa_decode(q, q_rope, ks[i % ROTATE], vs[i % ROTATE], flat[w.d_c:], bt, sl,
                           n_kv=w.n_kv, page_size=w.page_size, softmax_scale=w.scale,
                           causal=w.causal, rope_tok_stride=width, num_splits=args.num_splits,
                           seqlens_host=x["seqlens"], out=out, lse=lse, stream=stream,
                           kernel_events=events)

    def oracle_seqs(seqs, rows):
        """fp64 expansion of just the tokens of sequences `seqs` (their pages
        copied into a compact pool), then grouped decode of `rows` (flat row
        ids within that compact batch)."""
        pages = [x["block_table"][s, : (int(x["seqlens"][s]) + P - 1) // P] for s in seqs]
        sub_bt = np.full((len(seqs), x["block_table"].shape[1]), -1, np.int32)
        pool = []
        for i, pg in enumerate(pages):
            sub_bt[i, : len(pg)] = np.arange(len(pool), len(pool) + len(pg))
            pool.extend(pg.tolist())
        sub_kv = x["kv"][np.array(pool)]
        sub_sl = x["seqlens"][seqs]
        rk, rv = oracle.expand_latent(sub_kv.reshape(-1), f64(x["w_uk"]), f64(x["w_uv"]), sub_bt,
                                      sub_sl, page_size=P, num_pages=len(pool),
                                      kv_tok_stride=width)
        return oracle.gqa_decode(f64(x["q_nope_h"])[seqs], np.nan_to_num(rk), np.nan_to_num(rv),
                                 sub_bt, sub_sl, n_kv=w.n_kv, d_h=w.d_h, page_size=P,
                                 scale=w.scale, causal=w.causal, q_rope=f64(x["q_rope"])[seqs],
                                 k_rope=np.nan_to_num(f64(sub_kv[..., w.d_c:])), d_rope=w.d_rope,
                                 rows=rows)

    def parity():
        per = w.s_q * w.h_q
        seqs = [0, w.B - 1]
        rng = np.random.default_rng(13)
        sub_rows = np.sort(np.concatenate(
            [i * per + rng.choice(per, 8, replace=False) for i in range(len(seqs))])).astype(np.int32)
        rows = np.array([seqs[int(r) // per] * per + int(r) % per for r in sub_rows])
        ro, _ = oracle_seqs(seqs, sub_rows)
        got = out.float().cpu().numpy().reshape(-1, w.d_h)[rows]
        return rel_l2(got, ro.reshape(-1, w.d_h)[sub_rows])

    def cpu(budget):
        per = w.s_q * w.h_q
        done, el = timed_oracle(
            lambda s0, n: oracle_seqs(list(range(s0, s0 + n)), np.arange(n * per, dtype=np.int32)),
            w.B, budget)
        return done, el, f"{seq_sample(done, w.B)}: fp64 latent expansion of their tokens " \
                         f"plus grouped decode of all {w.h_q} heads x {w.s_q} query tokens"

    work = rf.gqa_work(x["seqlens"], s_q=w.s_q, h_q=w.h_q, n_kv=w.n_kv, d_h=w.d_h,
                       d_rope=w.d_rope, page_size=w.page_size, causal=w.causal)

    # the steps on either side of absorbed decode, each timed on its own on
    # the same weights (not part of the timed step): W_UK into the query,
    # W_UV on the latent output, the step's new tokens into a copy of the
    # latent cache
    def timed_us(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    q_h = to_dev(x["q_nope_h"], torch)
    q_abs = lkv.lkv_absorb_query(q_h, wuk, stream=stream)
    o_up = torch.empty_like(q_h)
    kv_copy = kv.clone()
    P = w.page_size
    new_rows = torch.stack([torch.stack([kv[int(x["block_table"][b, j // P]), j % P]
                                         for j in range(int(L) - w.s_q, int(L))])
                            for b, L in enumerate(x["seqlens"])])
    rows = w.B * w.s_q * w.h_q
    wbytes = w.n_kv * w.d_c * w.d_h * 2
    t_abs = timed_us(lambda: lkv.lkv_absorb_query(q_h, wuk, out=q_abs, stream=stream))
    t_up = timed_us(lambda: lkv.lkv_up_project(q_abs, wuv, out=o_up, stream=stream))
    t_app = timed_us(lambda: lkv.lkv_append_tokens(new_rows, kv_copy, bt, sl, page_size=P,
                                                   stream=stream))
    proj_flops = 2.0 * rows * w.d_c * w.d_h
    proj_bytes = rows * (w.d_c + w.d_h) * 2 + wbytes
    app_bytes = 2 * w.B * w.s_q * width * 2
    del kv_copy
    n_tok = int(np.sum(x["seqlens"]))
    ew = rf.expand_work(n_tok, g=w.n_kv, d_c=w.d_c, d_h=w.d_h)
    ew8 = rf.expand_work(n_tok, g=w.n_kv, d_c=w.d_c, d_h=w.d_h, out_elem=1)
    extra = {"expansion": {"us": t_exp * 1e6, "tokens": n_tok, "algorithmic_bytes": ew.bytes,
                           "flops": ew.flops, "GB_per_s": ew.bytes / t_exp / 1e9,
                           "TFLOP_per_s": ew.flops / t_exp / 1e12,
                           "note": "cache-write-time expansion, not part of the timed step"},
             "expansion_e4m3": {"us": t_exp8 * 1e6, "algorithmic_bytes": ew8.bytes,
                                "GB_per_s": ew8.bytes / t_exp8 / 1e9,
                                "TFLOP_per_s": ew8.flops / t_exp8 / 1e12,
                                "note": "the same expansion written as 8-bit E4M3 caches"},
             "expansion_vendor_gemm": {"us": t_gemm * 1e6, "TFLOP_per_s": ew.flops / t_gemm / 1e12,
                                       "note": "context only: torch.matmul (hipBLASLt) on contiguous "
                                               "operands of the same product, no gather or scatter"},
             "absorb_query": {"us": t_abs, "flops": proj_flops, "bytes": proj_bytes,
                              "GB_per_s": proj_bytes / t_abs / 1e3,
                              "TFLOP_per_s": proj_flops / t_abs / 1e6},
             "up_project": {"us": t_up, "flops": proj_flops, "bytes": proj_bytes,
                            "GB_per_s": proj_bytes / t_up / 1e3,
                            "TFLOP_per_s": proj_flops / t_up / 1e6},
             "append_tokens": {"us": t_app, "bytes": app_bytes, "GB_per_s": app_bytes / t_app / 1e3,
                               "note": "per step, B * s_q new rows of the latent + RoPE cache"}}
    return dict(step=step, work=work, parity=parity, cpu=cpu, out=out, kernel="mfma_decode_kernel",
                extra=extra, config={"g": w.n_kv, "d_h": w.d_h, "d_rope": w.d_rope, "d_c": w.d_c})


SETUPS = {"mla": setup_mla, "gqa": setup_gqa, "gqla": setup_gqla}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the chip settles about 100 steps (10-20 ms) into a run of the headline
    # shape; a shorter warm-up times part of that transient
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--workload", default="dsv3_mla_b64_l4096")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--ramp", type=int, default=0,
                    help="per-step times of a copy and of the step from a cold start, N steps each")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.steps if args.steps != 200 else 5)
        return
    if args.ramp:
        ramp(args.workload, args.ramp)
        return

    import torch
    import latent_kv_decode_amd as lkv
    import lkv_inputs as li
    from latent_kv_decode_amd import roofline as rf

    lkv.load_library()
    w = li.workload(args.workload)
    f32 = w.dtype == "f32"
    log(f"[bench] generating {w.name}")
    x = li.generate(w)
    s = SETUPS[w.kind](w, x, args, torch, lkv, rf)
    step, work = s["step"], s["work"]

    hip = HipEvents()
    ev_every = 4
    kev = [(hip.create(), hip.create()) for _ in range((args.steps + ev_every - 1) // ev_every)]
    stream = torch.cuda.current_stream()
    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(i, kev[i // ev_every] if i % ev_every == 0 else None)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span = e_start.elapsed_time(e_end) * 1e-3  # seconds, K steps
    kern = np.array([hip.elapsed_ms(a, b) for a, b in kev]) * 1e-3
    # the spread of single steps, from a second (untimed) pass with an event
    # pair per step; events between steps add their own small gaps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)]) * 1e-3
    for a, b in kev:
        hip.destroy(a)
        hip.destroy(b)
    t_step = span / args.steps
    t_kern = float(kern.mean())

    tokens = w.B * w.s_q
    hbm = work.bytes / t_kern / 1e9
    tflops = work.flops / t_kern / 1e12
    log("[bench] parity sample against the oracle")
    rel = s["parity"]()
    result = {
        "metric": METRIC,
        "value": tokens / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if f32 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "seq_len": int(x["seqlens"].max()),
                   "total_cache_tokens": int(np.sum(x["seqlens"])), "s_q": w.s_q, "h_q": w.h_q,
                   **s["config"], "page_size": w.page_size, "table": w.table,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": hbm, "peak": rf.MI355X_HBM_GBPS, "unit": "GB/s",
                     "frac": hbm / rf.MI355X_HBM_GBPS, "traffic": measured_traffic(w.name)},
        # the float32 path runs on the vector ALUs (no MFMA): its arithmetic
        # is placed against the fp32 vector peak instead
        ("alu" if f32 else "mfma"): {
            "achieved": tflops, "unit": "TFLOP/s",
            "peak": rf.MI355X_FP32_TFLOPS if f32 else rf.MI355X_BF16_TFLOPS,
            "frac": tflops / (rf.MI355X_FP32_TFLOPS if f32 else rf.MI355X_BF16_TFLOPS)},
        "kernel": f"{s['kernel']} (attention, timed alone); a step adds the split-KV combine "
                  "when a sequence spans several shares",
        "kernel_us": t_kern * 1e6,
        "kernel_timing": f"HIP events on the attention kernel of every {ev_every}th timed step "
                         f"({len(kev)} launches)",
        "kernel_us_median_p10_p90": [float(np.median(kern) * 1e6),
                                     float(np.percentile(kern, 10) * 1e6),
                                     float(np.percentile(kern, 90) * 1e6)],
        "step_us": t_step * 1e6,
        "step_us_median_p10_p90_single": [float(np.median(per) * 1e6), float(np.percentile(per, 10) * 1e6),
                                          float(np.percentile(per, 90) * 1e6)],
        "algorithmic": {"bytes_per_launch": work.bytes, "flops_per_launch": work.flops,
                        "intensity": work.intensity},
        "parity_sample_rel_l2": rel,
    }
    result["counters"] = counter_fields(w.name)
    result.update(s.get("extra", {}))
    if f32:
        result["note"] = ("a few kilobytes of cache per step: the kernel is bound by launch "
                          "latency, far from either roofline")
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] cpu baseline (fp64 oracle)")
        done, el, sample = s["cpu"](args.cpu_budget)
        result["cpu_baseline"] = {"value": done * w.s_q / el, "unit": "tokens/s",
                                  "cores": oracle.num_threads(), "kind": "oracle",
                                  "sample": f"{sample}; {el:.1f} s"}
        if f32:
            # the tiny workload also on one core
            cores = oracle.num_threads()
            oracle.set_num_threads(1)
            done1, el1, sample1 = s["cpu"](args.cpu_budget)
            oracle.set_num_threads(cores)
            result["cpu_baseline_single_core"] = {
                "value": done1 * w.s_q / el1, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"{sample1}; {el1:.1f} s"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
