#!/usr/bin/env python3
"""Benchmark: paged GQA decode step on one MI355X.

A step is one pass of the hot path over the batch-64 GQA serving-decode workload (B=64, H=32,
G=8, D=128, bs=16, past ~ U[512, 8192], seed 2): one pa_append_attention call, i.e. the append
of the 64 new K/V rows beside the device planner in one launch, then the split-KV decode kernel
and the log-sum-exp combine. Inputs are resident in HBM before timing starts. The same step as
two calls (pa_kv_append, then pa_paged_attention) is timed beside it.

Printed: ONE JSON line. `value` is the step's KV-cache read rate (sum_b L_b * G * D * 2 * 2
bytes per step / step time) in GB/s; `query_tokens_per_s` sits beside it. `roofline` is the
decode attention kernel alone: algorithmic KV bytes per launch / its mean launch time from HIP
events recorded by the library on the launch stream, against 8 TB/s. `cpu_baseline` times the
CPU oracle on the same workload's attention rows. `extra` carries the mixed prefill+decode and
block-sparse workloads. Beside the contract's mean over the timed steps: p10 / p50 / p90 of 100
individually timed steps, and the GPU's own 1 GiB device-copy rate (bytes read + written) as a
second reference next to the 8 TB/s peak.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFS = 2500.0
FLUSH_BYTES = 512 << 20  # written between launches of cache-sized workloads (> the 256 MB MALL)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip mixed and sparse workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run three 1 GiB device copies (for counter calibration runs)")
    return ap.parse_args()


# Sources that shape each profiled launch (its kernel code, the structs it reads and the host code
# that sizes its grid). A counter reading stays valid only while these files are unchanged.
KERNEL_SOURCES = {
    "attn_decode": ("attention.hip", "decode_unit.h", "plan.h", "common.h", "api.hip"),
    "prefill_combine": ("prefill.hip", "decode_unit.h", "combine_rows.h", "plan.h", "common.h",
                        "api.hip"),
    "decode_prefill": ("prefill.hip", "decode_unit.h", "combine_rows.h", "plan.h", "common.h",
                       "api.hip"),
    "append_plan": ("kv_append.hip", "plan.h", "common.h", "api.hip"),
    "kv_append": ("kv_append.hip", "common.h", "api.hip"),
    "plan": ("attention.hip", "plan.h", "common.h", "api.hip"),
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_gqa_paged_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on the current sources
    of that launch."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if k is None or k.get("source_hash") != kernel_source_hash(kernel):
        return None
    return k.get("bytes_per_launch")


def timed(fn, steps, warmup, torch, warm_ms=0.0):
    """Mean ms per step of `steps` steps, after at least `warmup` untimed steps and at least
    `warm_ms` of untimed work."""
    t_w = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t_w) * 1e3 < warm_ms:
        fn()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return s.elapsed_time(e) / steps, wall


def step_percentiles(fn, n, warmup, torch, np):
    """Per-step durations (ms) from an event pair around each of n steps: p10, p50, p90."""
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    t = np.array([s.elapsed_time(e) for s, e in ev])
    return {f"p{q}": round(float(np.percentile(t, q)), 4) for q in (10, 50, 90)}


def device_copy_gbps(torch, nbytes=1 << 30, reps=5):
    """The GPU's own device-to-device copy rate (bytes read + bytes written per second)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


WARM_MS = 100.0  # untimed work before each secondary workload's timed loop


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cold_kernel_us(pa, torch, fn, kernel, n, flush):
    """Mean duration (us) of the library launch `kernel` over n calls of fn, each preceded by a
    512 MB write that evicts the caches (only the kernel's own hook-timed interval is counted)."""
    pa.pa_timing_reset()
    for _ in range(n):
        flush.zero_()
        pa.pa_timing_enable(True)
        fn()
        pa.pa_timing_enable(False)
    torch.cuda.synchronize()
    t = pa.pa_timing_get(kernel)
    pa.pa_timing_reset()
    return t[0] / max(1, t[1]) * 1e3


def torch_kernel_us(torch, fn, n, flush=None):
    """Mean duration (us) of fn (torch work on the current stream), from an event pair around
    each call; with flush, a 512 MB write before each call (outside the timed pair)."""
    tot = 0.0
    for _ in range(n):
        if flush is not None:
            flush.zero_()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        tot += s.elapsed_time(e)
    return tot / n * 1e3


def oracle_all_cores(oracle, w, kc, vc, ref, kv, np):
    """The same oracle call on every host core: the batch is cut into contiguous groups of
    sequences, one per thread (the oracle runs in C, outside the interpreter lock), each group
    a workload of its own over the shared caches. The joined rows must equal the
    single-threaded result bit for bit."""
    import concurrent.futures as cf
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(16, cores, w["B"]))  # at most the 16 host cores of a one-GPU share
    cu = w["cu"]
    bounds = np.linspace(0, w["B"], cores + 1).astype(int)

    def part(k):
        b0, b1 = int(bounds[k]), int(bounds[k + 1])
        r0, r1 = int(cu[b0]), int(cu[b1])
        sub = dict(w)
        sub.update(B=b1 - b0, T=r1 - r0, cu=(cu[b0:b1 + 1] - cu[b0]).astype(np.int32),
                   past=w["past"][b0:b1], block_table=w["block_table"][b0:b1],
                   query=w["query"][r0:r1])
        return oracle.paged_attention(sub, kc, vc)

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        parts = list(ex.map(part, range(cores)))
    dt = time.perf_counter() - t0
    joined = np.concatenate(parts, axis=0)
    assert np.array_equal(joined.view(np.uint16), ref.view(np.uint16)), "partitioned oracle differs"
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"the same rows, {cores} threads over contiguous sequence groups, "
                      f"{dt:.2f} s", "host": host_cpu_model()}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_gqa_paged_amd as pa
    from block_sparse_gqa_paged_amd import device as dev
    from block_sparse_gqa_paged_amd import workloads as W

    torch.cuda.set_device(0)
    print("# generating the batch-64 GQA decode workload", file=sys.stderr, flush=True)
    w = W.gqa_decode()
    kv = W.kv_bytes(w)
    c = dev.PagedCase(w)

    def step():
        c.append_attention(pa.PA_SPLITS_AUTO)

    def step_two_calls():
        c.append()
        c.attention(pa.PA_SPLITS_AUTO)

    pa.pa_timing_reset()
    pa.pa_timing_enable(True)
    ms, wall = timed(step, args.steps, args.warmup, torch)
    pa.pa_timing_enable(False)
    kt = {k: pa.pa_timing_get(k) for k in ("append_plan", "attn_decode", "prefill_combine")}
    pa.pa_timing_reset()
    # the same steps without the library's event records, for the step time itself
    ms_plain, _ = timed(step, args.steps, args.warmup, torch)
    ms_two, _ = timed(step_two_calls, args.steps, args.warmup, torch)
    # the manifest's own split rule (numSplits from MAX_SPLITS / SPLIT_MIN_KEYS /
    # SPLIT_TARGET_WORKGROUPS: S = 2 here) through the same one-call step
    ms_page, _ = timed(lambda: c.append_attention(pa.PA_SPLITS_PAGE_RULE), args.steps,
                       args.warmup, torch)
    pct = step_percentiles(step, 100, 10, torch, np)
    copy_gbps = device_copy_gbps(torch)
    print(f"# step {ms_plain:.4f} ms (with event hooks {ms:.4f} ms; as two calls {ms_two:.4f} ms)",
          file=sys.stderr, flush=True)

    dec_ms = kt["attn_decode"][0] / max(1, kt["attn_decode"][1])
    achieved = kv / (dec_ms * 1e-3) / 1e9
    value = kv / (ms_plain * 1e-3) / 1e9
    per_kernel = {k: round(v[0] / max(1, v[1]) * 1e3, 2) for k, v in kt.items() if v[1]}

    cpu = cpu_all = None
    if not args.no_cpu:
        import oracle
        print("# timing the CPU oracle on the same attention rows", file=sys.stderr, flush=True)
        kc = c.key_cache.cpu().numpy()
        vc = c.value_cache.cpu().numpy()
        t0 = time.perf_counter()
        ref = oracle.paged_attention(w, kc, vc)
        dt = time.perf_counter() - t0
        cpu = {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"all {w['T']} decode rows x {w['H']} heads of the workload, "
                         f"attention only, {dt:.1f} s single-threaded",
               "host": host_cpu_model()}
        cpu_all = oracle_all_cores(oracle, w, kc, vc, ref, kv, np)

    extra = {}
    if not args.no_extra:
        extra = run_extra(args, torch, np, pa, dev, W)
    if args.copy_calibration:
        # kernels of known traffic, for scaling HBM counter readings: a plain device copy, and
        # as an independent check a reduction that only reads and a fill that only writes
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        total = float(src.sum().item())
        dst.fill_(2.0)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes_each_way"] = src.numel() * 4
        extra["read_calibration_sum"] = total

    line = {
        "metric": "paged-attn decode KV GB/s (% of HBM peak) and query tokens/s, 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "query_tokens_per_s": round(w["T"] / (ms_plain * 1e-3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_plain, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w["name"], "batch": w["B"], "num_heads": w["H"],
                   "kv_num_heads": w["G"], "head_size": w["D"], "block_size": w["bs"],
                   "past_seqlens": "uniform [512, 8192], seed 2", "kv_bytes_per_step": kv,
                   "num_splits": "auto", "parallelism": "none (1 GPU)"},
        "kernel_us": per_kernel,
        "two_calls_ms_per_step": round(ms_two, 4),
        "page_rule_splits_ms_per_step": round(ms_page, 4),
        "page_rule_splits_pct_of_hbm_peak": round(100.0 * kv / (ms_page * 1e-3) / 1e9
                                                  / HBM_PEAK_GBS, 2),
        "step_ms_percentiles_100": pct,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles("attn_decode"),
                     "kernel": "attn_decode", "kernel_us": round(dec_ms * 1e3, 2),
                     "device_copy_GBps_read_plus_write": copy_gbps},
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def run_extra(args, torch, np, pa, dev, W):
    out = {}
    steps = max(3, args.steps // 5)
    # Untimed work before each timed loop. The compute-bound prefill runs up to 25% slower for
    # the first few tens of milliseconds after the memory-bound decode loop (130-134 us, then
    # 106-107 us on the mixed workload), so each secondary loop warms up for 100 ms of its own.
    wu = max(10, args.warmup)

    def warm(fn):  # untimed, with the library's timing hooks off
        timed(fn, 1, wu, torch, WARM_MS)
    # Workloads smaller than the 256 MB last-level cache are timed cold: a 512 MB write before
    # each launch evicts their inputs (the write itself is not timed).
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    n_cold = max(5, steps)
    print("# generating the mixed prefill+decode workload", file=sys.stderr, flush=True)
    w = W.mixed_prefill_decode()
    c = dev.PagedCase(w)
    kv = W.kv_bytes(w)
    warm(lambda: (c.append(), c.attention(pa.PA_SPLITS_AUTO)))
    pa.pa_timing_reset()
    pa.pa_timing_enable(True)
    ms, _ = timed(lambda: (c.append(), c.attention(pa.PA_SPLITS_AUTO)), steps, 0, torch)
    pa.pa_timing_enable(False)
    kt = {k: pa.pa_timing_get(k) for k in ("kv_append", "plan", "attn_decode", "prefill_combine",
                                           "decode_prefill", "combine")}
    pa.pa_timing_reset()
    ms_one, _ = timed(lambda: c.append_attention(pa.PA_SPLITS_AUTO), steps, wu, torch, WARM_MS)
    us = {k: round(v[0] / max(1, v[1]) * 1e3, 2) for k, v in kt.items() if v[1]}
    # prefill flops: causal QK^T and PV over the prefill rows, 4*D per (row, head, key)
    L = w["past"].astype(np.int64)
    n = np.diff(w["cu"]).astype(np.int64)
    flops = 0
    for b in range(w["B"]):
        if n[b] > 1:
            keys = L[b] + np.arange(1, n[b] + 1)
            flops += int(keys.sum()) * w["H"] * w["D"] * 4
    # The decode and prefill items of this call share one launch; the prefill alone is timed on
    # the same 8 prefill sequences without the decode rows (the same prefill items, the whole
    # machine to themselves).
    wp = W.mixed_prefill_decode(n_decode=0)
    cp = dev.PagedCase(wp)
    warm(lambda: (cp.append(), cp.attention(pa.PA_SPLITS_AUTO)))
    pa.pa_timing_reset()
    pa.pa_timing_enable(True)
    timed(lambda: cp.attention(pa.PA_SPLITS_AUTO), steps, 0, torch)
    pa.pa_timing_enable(False)
    t_pre = pa.pa_timing_get("decode_prefill")
    pa.pa_timing_reset()
    us_pre = t_pre[0] / max(1, t_pre[1]) * 1e3
    del cp
    app_bytes = w["T"] * w["G"] * w["D"] * 2 * 4 + w["T"] * (w["rotary_dim"] // 2) * 2 * 2
    out["mixed_prefill_decode"] = {
        "workload": w["name"], "ms_per_step": round(ms, 4),
        "one_call_ms_per_step": round(ms_one, 4), "kernel_us": us,
        "kv_bytes": kv, "step_kv_GBps": round(kv / (ms * 1e-3) / 1e9, 1),
        "prefill_alone_us": round(us_pre, 2),
        "prefill_TFLOPs": round(flops / (us_pre * 1e-6) / 1e12, 2),
        "prefill_mfma_frac": round(flops / (us_pre * 1e-6) / 1e12 / MFMA_F16_PEAK_TFS, 4),
        "prefill_flops": flops,
        "append_GBps": round(app_bytes / (us.get("kv_append", 1e9) * 1e-6) / 1e9, 1),
        "append_pct_hbm": round(100 * app_bytes / (us.get("kv_append", 1e9) * 1e-6) / 1e9
                                / HBM_PEAK_GBS, 2),
        "append_bytes": app_bytes,
        "append_cache": "in the step: the previous step's 1.8 GB decode has evicted its inputs",
    }
    # What a 35 MB append can reach on this machine: the same append cold (flush before each
    # launch), a plain device copy moving the same bytes (half read, half written) cold, and the
    # append of 2 tokens (one workgroup: the launch and its dependent loads, no bandwidth).
    us_cold = cold_kernel_us(pa, torch, c.append, "kv_append", n_cold, flush)
    src = torch.empty(app_bytes // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    us_copy = torch_kernel_us(torch, lambda: dst.copy_(src), n_cold, flush)
    del src, dst
    w2 = W.paged_workload(7, past=[100], n_new=[2], num_heads=32, kv_num_heads=8,
                          head_size=128, block_size=32, packed=True, rotary_mode=W.ROTARY_NEOX,
                          rotary_dim=128, rotary_positions=256, name="append_2_tokens")
    c2 = dev.PagedCase(w2)
    warm(c2.append)
    us_min = cold_kernel_us(pa, torch, c2.append, "kv_append", n_cold, flush)
    del c2
    out["append_floor"] = {
        "workload": w["name"], "append_bytes": app_bytes,
        "append_cold_us": round(us_cold, 2),
        "append_cold_pct_hbm": round(100 * app_bytes / (us_cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "device_copy_same_bytes_cold_us": round(us_copy, 2),
        "device_copy_same_bytes_pct_hbm": round(100 * app_bytes / (us_copy * 1e-6) / 1e9
                                                / HBM_PEAK_GBS, 2),
        "append_2_tokens_us": round(us_min, 2),
        "us_at_60pct_hbm": round(app_bytes / (0.6 * HBM_PEAK_GBS * 1e9) * 1e6, 2),
    }
    # the append with every new query row rotated into q_out in the same launch
    q_out = torch.empty((w["T"], w["H"] * w["D"]), dtype=torch.float16, device="cuda")
    warm(lambda: c.append_rotate_query(q_out))
    us_rq = cold_kernel_us(pa, torch, lambda: c.append_rotate_query(q_out), "kv_append", n_cold,
                           flush)
    rq_bytes = app_bytes + w["T"] * w["H"] * w["D"] * 2 * 2
    out["mixed_prefill_decode"].update({
        "append_rotate_query_us": round(us_rq, 2), "append_rotate_query_bytes": rq_bytes,
        "append_rotate_query_GBps": round(rq_bytes / (us_rq * 1e-6) / 1e9, 1),
        "append_rotate_query_cache": "cold (512 MB written before each launch)"})
    del c, q_out
    torch.cuda.empty_cache()

    # the append alone at 16x the mixed workload's prefill tokens: its bandwidth regime
    print("# generating the append stress workload", file=sys.stderr, flush=True)
    w = W.append_stress()
    c = dev.PagedCase(w)
    warm(c.append)
    pa.pa_timing_reset()
    pa.pa_timing_enable(True)
    ms, _ = timed(c.append, steps, 0, torch)
    pa.pa_timing_enable(False)
    t_app = pa.pa_timing_get("kv_append")
    pa.pa_timing_reset()
    us_app = t_app[0] / max(1, t_app[1]) * 1e3
    app_bytes = w["T"] * w["G"] * w["D"] * 2 * 4 + w["T"] * (w["rotary_dim"] // 2) * 2 * 2
    out["append_stress"] = {
        "workload": w["name"], "tokens": w["T"], "append_bytes": app_bytes,
        "kernel_us": round(us_app, 2), "append_GBps": round(app_bytes / (us_app * 1e-6) / 1e9, 1),
        "pct_hbm": round(100 * app_bytes / (us_app * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
    }
    del c
    torch.cuda.empty_cache()

    # the append page's own pass: contiguous BNSH cache, padded batch
    print("# generating the contiguous-cache append workload", file=sys.stderr, flush=True)
    bw = W.bnsh_append()
    bc = dev.BnshCase(bw)
    warm(bc.append)
    us_b = cold_kernel_us(pa, torch, bc.append, "kv_append_bnsh", n_cold, flush)
    rows = bw["B"] * bw["S"]
    b_bytes = rows * bw["KVH"] * bw["D"] * 2 * 4 + rows * (bw["rotary_dim"] // 2) * 2 * 2
    out["append_bnsh"] = {
        "workload": bw["name"], "append_bytes": b_bytes, "kernel_us": round(us_b, 2),
        "append_GBps": round(b_bytes / (us_b * 1e-6) / 1e9, 1),
        "pct_hbm": round(100 * b_bytes / (us_b * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "cache": "cold (512 MB written before each launch)",
    }
    del bc
    torch.cuda.empty_cache()

    print("# generating the block-sparse workload", file=sys.stderr, flush=True)
    sw = W.block_sparse_forward()
    s = dev.SparseCase(sw)
    warm(lambda: (s.forward(), s.combine()))
    pa.pa_timing_reset()
    pa.pa_timing_enable(True)
    ms, _ = timed(lambda: (s.forward(), s.combine()), steps, 0, torch)
    pa.pa_timing_enable(False)
    kt = {k: pa.pa_timing_get(k) for k in ("sparse_forward", "combine")}
    pa.pa_timing_reset()
    us = {k: round(v[0] / max(1, v[1]) * 1e3, 2) for k, v in kt.items() if v[1]}
    # the edge list itself, built on the device from the kept-block mask
    eb = dev.EdgeBuilder(sw)
    warm(eb.build)
    us_edges = cold_kernel_us(pa, torch, eb.build, "build_edges", n_cold, flush)
    edge_bytes = sw["block_mask"].size + sw["E"] * 20 + (sw["Tq"] * sw["hkv"] + 1) * 4
    del eb
    # the same edges under the right-aligned causal mask
    warm(lambda: s.forward(causal=True))
    pa.pa_timing_reset()
    pa.pa_timing_enable(True)
    timed(lambda: s.forward(causal=True), steps, 0, torch)
    pa.pa_timing_enable(False)
    t_c = pa.pa_timing_get("sparse_forward")
    pa.pa_timing_reset()
    us_causal = t_c[0] / max(1, t_c[1]) * 1e3
    E, q, D = sw["E"], sw["qhead"], sw["D"]
    part_bytes = E * q * (D + 2) * 4
    rows = sw["Tq"] * sw["hq"]
    comb_bytes = part_bytes + rows * D * 4 + (len(sw["group_ptr"])) * 4
    # flops over mapped keys: 4*D per (edge lane, key)
    em = sw["edge_meta"]
    ppb = sw["pages_per_block"]
    mapped = (sw["block_tables"] >= 0)
    mk = 0
    blen = em[:, 4].astype(np.int64)
    for t in range(sw["block_size"]):
        ok = (blen > t) & mapped[em[:, 3], em[:, 2] * ppb + t // sw["page_size"]]
        mk += int(ok.sum())
    flops = mk * q * D * 4
    # the forward's own floor: writing its partials at the rate this device fills a buffer of
    # the same size
    wbuf = torch.empty(part_bytes, dtype=torch.uint8, device="cuda")
    us_fill = torch_kernel_us(torch, lambda: wbuf.fill_(1), n_cold)
    del wbuf
    fwd_us = us.get("sparse_forward", 1e9)
    out["block_sparse"] = {
        "workload": sw["name"], "edges": E, "ms_per_step": round(ms, 4), "kernel_us": us,
        "combine_GBps": round(comb_bytes / (us.get("combine", 1e9) * 1e-6) / 1e9, 1),
        "combine_bytes": comb_bytes,
        "combine_pct_hbm": round(100 * comb_bytes / (us.get("combine", 1e9) * 1e-6) / 1e9
                                 / HBM_PEAK_GBS, 2),
        "forward_flops": flops,
        # it runs fp16 matrix instructions: three fp16 products per fp32 product
        "forward_fp32_TFLOPs": round(flops / (fwd_us * 1e-6) / 1e12, 2),
        "forward_frac_f16_mfma_algorithmic": round(flops / (fwd_us * 1e-6) / 1e12
                                                   / MFMA_F16_PEAK_TFS, 4),
        "forward_frac_f16_mfma_executed": round(3 * flops / (fwd_us * 1e-6) / 1e12
                                                / MFMA_F16_PEAK_TFS, 4),
        # its bound: the partial writes (E * qhead * (D + 2) * 4 bytes)
        "partial_bytes": part_bytes,
        "partial_write_floor_us": round(us_fill, 2),
        "forward_vs_write_floor": round(us_fill / fwd_us, 4),
        "partial_write_frac_hbm_peak": round(part_bytes / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                             4),
        "causal_forward_us": round(us_causal, 2),
        "build_edges_us": round(us_edges, 2), "build_edges_bytes": edge_bytes,
        "build_edges_GBps": round(edge_bytes / (us_edges * 1e-6) / 1e9, 1),
        "build_edges_cache": "cold (512 MB written before each launch)",
    }
    return out


if __name__ == "__main__":
    main()
