#!/usr/bin/env python3
"""Benchmark of the shared-round attention hot path on one MI355X.

Default workload: 16 one-row decode streams, 32 query / 8 kv heads, head dim
128, key counts uniform in [512, 4096] in 32-token pages scattered over a
4096-page pool, split-K 512 keys a partial + merge.  One step = tf_attn_rows
+ tf_attn_merge over every stream (workloads with logits add tf_argmax).

Inputs are resident in HBM before timing starts.  The K/V pool is kept in
``--copies`` copies (each with its own segment table) and the steps rotate
over them, so that K/V is read from HBM and not from the 256 MB Infinity
Cache.  Printed: one JSON line: metric, value = KV-read GB/s of the whole
step over exactly --steps steps, the step's median / p10 / p90 over
--dist-steps steps timed one by one, the roofline of the rows kernel, a
measured device-copy ceiling, a side table with the other four workloads
(attention step and argmax, each timed step by step, with its roofline
fraction), and the CPU oracle's rate on every host core and on one core,
with the CPU model.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak

METRIC = "KV-read GB/s (% of HBM peak) and attn rows/s, 16-stream decode"
PMC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kv_bytes(w) -> int:
    """Algorithmic bytes: each visible key's K and V once, all kv heads."""
    return sum(s.key_count for s in w.segments) * w.n_kv_heads * w.head_dim * 2 * 2


def attn_flops(w) -> int:
    """QK^T and P.V multiply-adds (2 flops each) over every row's visible keys."""
    total = 0
    for s in w.segments:
        vis = sum(s.key_count - s.n_rows + r + 1 for r in range(s.n_rows))
        total += vis * w.n_q_heads * w.head_dim * 2 * 2
    return total


def traffic_entry(name: str):
    """HBM bytes per rows launch from the committed rocprofv3 counter runs, or None
    when the kernel source changed since they were taken."""
    try:
        with open(PMC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    from stream_paged_attention_amd.profsum import kernel_hash
    e = data.get(name)
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(w, budget_s: float, threads: int):
    """Run the oracle over the whole workload (or a row sample of the prompt
    chunk) repeatedly for about budget_s; rates from the median repetition."""
    from oracle import oracle
    rows = None
    if w.name == "prompt512":      # bounded sample: a few rows of the prompt chunk
        rows = [0, 128, 256, 384, 511]
    times, used = [], threads
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        _, used = oracle.attn_workload(w, rows=rows, threads=threads, return_threads=True)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end and len(times) >= 3:
            break
    med = sorted(times)[len(times) // 2]
    if rows is None:
        nbytes, nrows = kv_bytes(w), w.total_rows
        sample = f"whole workload, median of {len(times)} runs ({sum(times):.1f} s)"
    else:
        seg = w.segments[0]
        nbytes = sum(seg.key_count - seg.n_rows + r + 1 for r in rows) * w.n_kv_heads * w.head_dim * 4
        nrows = len(rows)
        sample = f"{len(rows)} of {w.total_rows} rows, median of {len(times)} runs ({sum(times):.1f} s)"
    return {"value": round(nbytes / med / 1e9, 4), "unit": "GB/s", "cores": int(used),
            "kind": "oracle", "sample": sample, "rows_per_s": round(nrows / med, 2),
            "median_s": round(med, 5)}


def cpu_baseline(w, budget_s: float):
    """The float64 oracle on every host core, and again on one core."""
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))
    out = _oracle_rate(w, budget_s, threads)
    one = _oracle_rate(w, max(3.0, budget_s / 3), 1)
    out["cpu_model"] = cpu_model()
    out["nproc"] = os.cpu_count()
    out["one_core"] = {k: one[k] for k in ("value", "cores", "sample", "rows_per_s", "median_s")}
    return out


def bench_kv_put(args, w, dw, copies, stream) -> int:
    """tf_kv_put of every segment's round rows (its last n_rows keys), timed
    back to back; bytes = the rows' K and V read once and written once."""
    import numpy as np
    import torch
    from stream_paged_attention_amd import binding, synth
    rng = np.random.Generator(np.random.PCG64(synth.WORKLOAD_SEED[args.workload] + 100))
    shape = (w.total_rows, w.n_kv_heads, w.head_dim)
    k_new = torch.from_numpy(rng.integers(0, 1 << 16, size=shape, dtype=np.uint16).view(np.int16)).to(dw.device)
    v_new = torch.from_numpy(rng.integers(0, 1 << 16, size=shape, dtype=np.uint16).view(np.int16)).to(dw.device)
    st = stream.cuda_stream
    argl = [dw.put_args(k_new, v_new, c) for c in range(copies)]
    for i in range(args.warmup):
        assert binding.tf_kv_put(argl[i % copies], st) == 0
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        binding.tf_kv_put(argl[i % copies], st)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    assert dw.error_word() == 0
    nbytes = 2 * 2 * w.total_rows * w.n_kv_heads * w.head_dim * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": f"KV-append GB/s, synthetic workload {args.workload}", "value": round(gbps, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": synth.WORKLOAD_TITLES[args.workload] + " (round rows appended)", "rows": w.total_rows,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "bytes_per_step": nbytes,
                   "rows_per_s": round(w.total_rows / (ms * 1e-3), 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": "tf_kv_put (kv_put_kernel)"},
    }), flush=True)
    return 0


def bench_state(args) -> int:
    """tf_state_save and tf_state_restore of a kept state: ten layers' K and V
    at positions [0, 6243) (8 KV heads x D 64, 512-position pages of a
    shuffled page list), alternating between two disjoint page lists and two
    state buffers so that the working set exceeds the last-level cache.  Bytes
    per call = what is read plus what is written."""
    import ctypes
    import numpy as np
    import torch
    from stream_paged_attention_amd import binding
    dev = torch.device("cuda:0")
    layers, hkv, d, page, at, pool_pages = 10, 8, 64, 512, 6243, 32
    n_state = -(-at // page)
    gen = torch.Generator(device=dev)
    gen.manual_seed(6243)
    rnd = lambda *shape: torch.randint(-32768, 32767, shape, dtype=torch.int16, device=dev, generator=gen)
    pools = [(rnd(pool_pages, hkv, page, d), rnd(pool_pages, hkv, page, d)) for _ in range(layers)]
    states = [[(rnd(n_state, hkv, page, d), rnd(n_state, hkv, page, d)) for _ in range(layers)] for _ in range(2)]
    perm = np.random.Generator(np.random.PCG64(6243)).permutation(pool_pages).astype(np.int32)
    page_lists = [torch.from_numpy(perm[i * n_state:(i + 1) * n_state].copy()).to(dev) for i in range(2)]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    keep = []
    argl = []
    for c in range(2):
        table = (binding.tf_state_layer * layers)()
        for i in range(layers):
            table[i].pool_k, table[i].pool_v = pools[i][0].data_ptr(), pools[i][1].data_ptr()
            table[i].state_k, table[i].state_v = states[c][i][0].data_ptr(), states[c][i][1].data_ptr()
        raw = bytes(ctypes.string_at(ctypes.addressof(table), ctypes.sizeof(table)))
        t = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(dev)
        keep.append(t)
        a = binding.tf_state_args()
        a.n_layers, a.n_kv_heads, a.head_dim, a.page_size, a.pool_pages = layers, hkv, d, page, pool_pages
        a.at, a.n_pages, a.pages, a.layers, a.err = at, n_state, page_lists[c].data_ptr(), t.data_ptr(), err.data_ptr()
        argl.append(a)
    st = torch.cuda.current_stream(dev).cuda_stream
    nbytes = 2 * layers * 2 * at * hkv * d * 2
    res = {}
    for name, fn in (("save", binding.tf_state_save), ("restore", binding.tf_state_restore)):
        for i in range(args.warmup):
            assert fn(argl[i % 2], st) == 0
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(args.steps):
            fn(argl[i % 2], st)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        res[name] = (ms, nbytes / (ms * 1e-3) / 1e9)
    assert int(err.item()) == 0
    gbps = res["save"][1]
    print(json.dumps({
        "metric": "kept-state copy GB/s (read + written), save", "value": round(gbps, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["save"][0], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "kept state of a 6,243-position history: 10 layers' K and V, 8 KV heads x D 64, "
                               "512-position pages of a shuffled page list",
                   "bytes_per_call": nbytes, "restore_ms": round(res["restore"][0], 5),
                   "restore_gbps": round(res["restore"][1], 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "tf_state_save (state_copy_kernel)",
                     "restore_frac": round(res["restore"][1] / HBM_PEAK_GBPS, 4)},
    }), flush=True)
    return 0


def percentiles(xs):
    """(median, p10, p90) of a list of floats."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return float(np.median(a)), float(np.percentile(a, 10)), float(np.percentile(a, 90))


class AttnStep:
    """One workload resident on the device: its K/V copies, tables, logits and
    the step (tf_attn_rows, tf_attn_merge when split, tf_argmax when the
    workload has logits) on the current stream."""

    def __init__(self, name: str, dev, copies: int = 0):
        import torch
        from stream_paged_attention_amd import binding, launch, synth
        self.binding = binding
        self.name = name
        self.w = w = synth.make_synthetic(name)
        self.copies = copies or max(1, min(8, -(-(2 * 256 * 2 ** 20) // max(1, kv_bytes(w)))))
        self.dw = launch.DeviceWorkload(w, dev, copies=self.copies)
        self.stream = torch.cuda.current_stream(dev)
        self.st = self.stream.cuda_stream
        self.argl = [self.dw.args(c) for c in range(self.copies)]
        self.split = self.dw.split_keys > 0
        self.logits = None
        if w.logits is not None:
            self.logits = launch._dev(w.logits, dev)
            self.nrows, self.vocab = w.logits.shape
            self.ids = torch.empty(self.nrows, dtype=torch.int32, device=dev)
            self.flags = torch.empty(self.nrows, dtype=torch.uint8, device=dev)
            self.wsb = binding.tf_argmax_workspace_bytes(self.nrows, self.vocab)
            self.ws = torch.zeros(self.wsb // 8 + 1, dtype=torch.int64, device=dev)   # zero before first use

    def attn(self, i: int) -> int:
        a = self.argl[i % self.copies]
        rc = self.binding.tf_attn_rows(a, self.st)
        if self.split:
            rc |= self.binding.tf_attn_merge(a, self.st)
        return rc

    def rows_only(self, i: int) -> int:
        return self.binding.tf_attn_rows(self.argl[i % self.copies], self.st)

    def argmax(self, i: int) -> int:
        return self.binding.tf_argmax(self.logits.data_ptr(), self.nrows, self.vocab, self.vocab,
                                      self.ids.data_ptr(), self.flags.data_ptr(), self.ws.data_ptr(),
                                      self.wsb, self.st)

    def full(self, i: int) -> int:
        rc = self.attn(i)
        if self.logits is not None:
            rc |= self.argmax(i)
        return rc

    def time_total(self, fn, steps: int, warmup: int) -> float:
        """Mean microseconds per call over exactly `steps` calls between one event pair."""
        import torch
        for i in range(warmup):
            assert fn(i) == 0
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for i in range(steps):
            fn(i)
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / steps

    def time_each(self, fn, steps: int, warmup: int):
        """Per-call microseconds: an event before every call and after the last."""
        import torch
        for i in range(warmup):
            assert fn(i) == 0
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for i in range(steps):
            ev[i].record(self.stream)
            fn(i)
        ev[steps].record(self.stream)
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps)]

    def error_word(self) -> int:
        return self.dw.error_word()


def copy_ceiling_gbps(dev, mib: int = 1024, reps: int = 10) -> float:
    """Bytes read plus bytes written per second by a plain device-to-device copy."""
    import torch
    x = torch.ones(mib << 20, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    s = a.elapsed_time(b) * 1e-3 / reps
    del x, y
    torch.cuda.empty_cache()
    return 2 * (mib << 20) / s / 1e9


def workload_entry(ws: "AttnStep", n_dist: int) -> dict:
    """Per-step distribution and roofline fraction of one workload's attention
    (and argmax), for the side table of the bench line."""
    w = ws.w
    kvb, flops = kv_bytes(w), attn_flops(w)
    med, p10, p90 = percentiles(ws.time_each(ws.attn, n_dist, 10))
    rows_us = ws.time_total(ws.rows_only, n_dist, 10)
    e = {"attn_us_median": round(med, 3), "attn_us_p10": round(p10, 3), "attn_us_p90": round(p90, 3),
         "rows_kernel_us": round(rows_us, 3), "kv_bytes": kvb, "attn_flops": flops,
         "value_gbps": round(kvb / (med * 1e-6) / 1e9, 2),
         "rows_per_s": round(w.total_rows / (med * 1e-6), 1),
         "hbm_frac": round(kvb / (rows_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
         "mfma_frac": round(flops / (rows_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    if ws.logits is not None:
        am, a10, a90 = percentiles(ws.time_each(ws.argmax, n_dist, 10))
        ak = ws.time_total(ws.argmax, n_dist, 10)   # back to back, like rows_kernel_us
        lb = ws.nrows * ws.vocab * 2
        e.update({"argmax_us_median": round(am, 3), "argmax_us_p10": round(a10, 3),
                  "argmax_us_p90": round(a90, 3), "argmax_kernel_us": round(ak, 3), "argmax_logit_bytes": lb,
                  "argmax_hbm_frac": round(lb / (ak * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                  "step_us_mean": round(ws.time_total(ws.full, n_dist, 10), 3)})
    if w.name == "prompt512":
        e["bound"] = "mfma"
    elif w.name == "single64":
        e["bound"] = "latency"
    else:
        e["bound"] = "hbm"
    assert ws.error_word() == 0
    return e


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode16",
                    choices=["single64", "decode16", "verify8", "prompt512", "ring17"],
                    help="synthetic workload (decode16: the 16-stream decode the metric is quoted on)")
    ap.add_argument("--copies", type=int, default=0, help="K/V copies rotated (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the other workloads' side table and the copy ceiling")
    ap.add_argument("--dist-steps", type=int, default=200,
                    help="steps timed one by one for the median and p10/p90 (at least 100)")
    ap.add_argument("--kernel-only", action="store_true",
                    help="time only tf_attn_rows launches (for profiler runs)")
    ap.add_argument("--op", choices=["attn", "kv_put", "state"], default="attn",
                    help="kv_put: time tf_kv_put of the workload's round rows instead; "
                         "state: time tf_state_save / tf_state_restore of a kept state")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run 20 plain device copies of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by stream or by kv head with no exchange between GPUs)",
              file=sys.stderr)
        return 2
    args.dist_steps = max(100, args.dist_steps)

    import torch
    from stream_paged_attention_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_mib:
        x = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        for _ in range(20):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": x.numel(), "copies": 20}), flush=True)
        return 0
    binding.load()
    if args.op == "state":
        return bench_state(args)
    ws = AttnStep(args.workload, dev, args.copies)
    w, dw, copies = ws.w, ws.dw, ws.copies
    pool_bytes = (w.pool_k.nbytes * 2 if w.pool_k is not None
                  else sum(x.nbytes for x in w.store_k) * 2)
    if args.op == "kv_put":
        return bench_kv_put(args, w, dw, copies, ws.stream)
    step = ws.rows_only if args.kernel_only else ws.full

    # the timed region: exactly K steps between two events on the launch stream
    for i in range(args.warmup):
        assert step(i) == 0
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(ws.stream)
    for i in range(args.steps):
        step(i)
    end.record(ws.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    # the same step timed one by one (an event before each): median, p10, p90
    s_med, s_p10, s_p90 = percentiles(ws.time_each(step, args.dist_steps, 10))
    # the rows kernel alone: back-to-back launches between one event pair on
    # the launch stream (average launch duration, gaps included)
    rows_avg_ms = ws.time_total(ws.rows_only, min(args.steps, 1000), 10) * 1e-3
    assert ws.error_word() == 0

    from stream_paged_attention_amd.profsum import kernel_hash as kernel_hash_now
    kvb = kv_bytes(w)
    flops = attn_flops(w)
    value = kvb / (ms_step * 1e-3) / 1e9
    achieved_hbm = kvb / (rows_avg_ms * 1e-3) / 1e9
    # the prompt chunk is a dense contraction on the matrix cores; the decode,
    # verify and ring workloads read each key once and are bound by HBM
    if args.workload == "prompt512":
        bound, ach, peak, unit = "mfma", flops / (rows_avg_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        kernel = "tf_attn_rows (rows_mfma_kernel)"
    else:
        bound, ach, peak, unit = "hbm", achieved_hbm, HBM_PEAK_GBPS, "GB/s"
        kernel = "tf_attn_rows (rows_valu_kernel)" if args.workload in ("single64", "decode16") else \
            "tf_attn_rows (rows_mfma_kernel + rows_valu_kernel)"
    traffic = traffic_entry(args.workload)
    out = {
        "metric": METRIC if args.workload == "decode16" else
        f"KV-read GB/s and attn rows/s, synthetic workload {args.workload}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": synth.WORKLOAD_TITLES[args.workload],
            "streams": len(w.segments), "rows": w.total_rows, "q_heads": w.n_q_heads,
            "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "page_size": w.page_size,
            "split_keys": dw.split_keys, "kv_bytes_per_step": kvb, "attn_flops_per_step": flops,
            "accumulate": "fp32", "kv_copies_rotated": copies, "pool_bytes_per_copy": pool_bytes,
            "rows_per_s": round(w.total_rows / (ms_step * 1e-3), 1),
            "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
            "step_us_median": round(s_med, 3), "step_us_p10": round(s_p10, 3),
            "step_us_p90": round(s_p90, 3), "dist_steps": args.dist_steps,
            "rows_kernel_us": round(rows_avg_ms * 1e3, 3),
            "wall_s": round(wall, 3),
            "kernel_hash": kernel_hash_now(),
        },
        "roofline": {"bound": bound, "achieved": round(ach, 3), "peak": peak, "unit": unit,
                     "frac": round(ach / peak, 4), "traffic": traffic,
                     "kernel": kernel,
                     "hbm_gbps_rows_kernel": round(achieved_hbm, 2)},
    }
    if not args.no_side and not args.kernel_only:
        out["copy_ceiling_gbps"] = round(copy_ceiling_gbps(dev), 1)
        side = {}
        for name in synth.WORKLOADS:
            if name == args.workload:
                continue
            other = AttnStep(name, dev)
            side[name] = workload_entry(other, args.dist_steps)
            del other
            torch.cuda.empty_cache()
        out["workloads"] = side
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
