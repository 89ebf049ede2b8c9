#!/usr/bin/env python3
"""Benchmark of the exact attention forward (fa_fwd) on one MI355X.

A step is one fa_fwd call over the whole batch of the headline workload
(B=2, H=16, N=4096, d=64, fp16, non-causal, scale 1/8): the complete hot path
(Q-tile pinning, K/V streaming, both MFMA GEMMs, online softmax, masking,
epilogue). Inputs are resident in HBM before timing starts.

Prints ONE JSON line. ``value`` is TFLOP/s counting 4*B*H*N^2*d (halved for causal).
``roofline`` prices the kernel against the dense fp16/bf16 MFMA peak, using the
per-launch duration measured with HIP events on the stream the kernel runs on.
``cpu_baseline`` times the fp64 CPU oracle on the same inputs (rank 0, N=1 only).
The other workloads are timed briefly and reported under ``other_workloads``.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

MFMA_PEAK_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk/CU (dense fp16/bf16) x 2.4 GHz
HBM_PEAK_GBS = 8000.0
HEADLINE = 2
# From idle, back-to-back launches of one kernel speed up over the first ~30-50 ms of
# device time before they reach a steady rate, which then holds (measured on MI355X:
# n4096_d64_f16 167 -> 141 us per launch over the first ~250 launches, then 140-142 us
# for 2.8 s, 20000 launches; n2048_d128_bf16_causal 186 -> 153 us). Every timing first
# runs its call for this much device time, so that the timed steps see the steady rate.
SETTLE_MS = 200.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="before the warm-up steps of each timing, run the timed call back to back "
                         "for at least this much device time (0: off); see settle()")
    ap.add_argument("--workload", type=int, default=HEADLINE, help="1..5 (default: the headline 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="turn two rocprofv3 --pmc runs of --profile (FETCH_SIZE, then WRITE_SIZE; "
                         "--output-format csv) into a calibrated per-launch HBM traffic record "
                         "(JSON on stdout); needs no GPU")
    ap.add_argument("--profile", action="store_true",
                    help="counter-collection mode: a few launches of --workload, then a plain "
                         "device copy of COPY_BYTES (read and written once) to calibrate the "
                         "HBM byte counters; prints one JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="with --profile: launch fa_bwd (after one fa_fwd for O and LSE) "
                         "instead of fa_fwd")
    return ap.parse_args()


COPY_BYTES = 1 << 30   # 1 GiB read + 1 GiB written by the calibration copy
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_forward_fwd_amd", *f) for f in
                  (("csrc", "fa_fwd.hip"), ("csrc", "fa_device.h"), ("build.py",))]
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    """SHA-256 over the forward kernels' sources (the kernel file, the device helpers it
    includes and the build script, which holds the compiler options)."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic_bytes(w) -> int:
    """Compulsory HBM bytes of one launch: Q, K, V read once, O written once (all in
    the 16-bit input type), LSE written once in fp32."""
    elems = w.B * w.H * w.N * w.d
    return 4 * elems * 2 + w.B * w.H * w.N * 4


def _pmc_rows(d, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    fa_vals, copy_vals = [], []
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            if "fa_fwd_kernel" in name or "fa_fwd_pipe_kernel" in name:
                fa_vals.append((name, float(row["Counter_Value"])))
            elif "copyBuffer" in name:
                copy_vals.append(float(row["Counter_Value"]))
    if not fa_vals or not copy_vals:
        raise SystemExit(f"{d}: missing attention-kernel or copy dispatches for {counter}")
    return fa_vals, copy_vals


def traffic_record(w, fetch_dir, write_dir):
    """Per-launch HBM bytes of the attention kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) each scaled by bytes / counter of a plain device copy of COPY_BYTES."""
    fa_f, cp_f = _pmc_rows(fetch_dir, "FETCH_SIZE")
    fa_w, cp_w = _pmc_rows(write_dir, "WRITE_SIZE")
    kib = lambda v: sum(v) / len(v)
    fetch_kib, write_kib = kib([v for _, v in fa_f]), kib([v for _, v in fa_w])
    copy_fetch_kib, copy_write_kib = kib(cp_f), kib(cp_w)
    f_fac = COPY_BYTES / (copy_fetch_kib * 1024)
    w_fac = COPY_BYTES / (copy_write_kib * 1024)
    hbm = fetch_kib * 1024 * f_fac + write_kib * 1024 * w_fac
    return {"workload": w.name, "kernel": fa_f[0][0], "kernel_source_sha256": kernel_source_hash(),
            "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
            "copy_bytes": COPY_BYTES, "copy_fetch_kib": copy_fetch_kib, "copy_write_kib": copy_write_kib,
            "fetch_factor": f_fac, "write_factor": w_fac, "hbm_bytes_per_launch": hbm,
            "algorithmic_bytes_per_launch": algorithmic_bytes(w),
            "traffic_over_algorithmic": hbm / algorithmic_bytes(w)}


def stored_traffic(w):
    """The committed traffic record for this workload, if it was taken on the current
    kernel source; else None."""
    path = os.path.join(PROFILES, f"traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec


def profile_mode(w, launches=3, backward=False):
    import torch
    import exact_attention_forward_fwd_amd as fa
    from exact_attention_forward_fwd_amd.workloads import make_inputs

    dev = torch.device("cuda:0")
    q, k, v, _ = make_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    tile = w.tile or (None, None)
    for _ in range(1 if backward else launches):
        fa.fwd(q, k, v, scale=w.scale, causal=w.causal, block_m=tile[0], block_n=tile[1], out=o, lse=lse)
    if backward:
        # dO as in the bench's backward timing
        g = torch.Generator("cpu").manual_seed(5000 + w.index)
        do = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
        for _ in range(launches):
            fa.bwd(q, k, v, o, do, lse, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(launches):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile": w.name, "backward": backward, "launches": launches, "copy_bytes": COPY_BYTES}),
          flush=True)


def settle(call, stream, min_ms, steps):
    """Runs `call` back to back in chunks of 16 until at least `min_ms` of device time has
    passed (one chunk stays queued while the previous one is checked, so the device
    never idles), then synchronises. Returns the launches and the device time. The
    launch count is kept different from `steps`, so that a kernel trace can tell this
    run from the timed one."""
    import torch

    if min_ms <= 0:
        return {"launches": 0, "ms": 0.0}
    chunk, n, total = 16, 0, 0.0
    start = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    prev = start
    pending = []
    while True:
        for _ in range(chunk):
            call()
        n += chunk
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        pending.append((prev, ev))
        prev = ev
        if len(pending) > 1:
            a, b = pending.pop(0)
            b.synchronize()
            total += a.elapsed_time(b)
            if (total >= min_ms and n != steps) or n >= 20000:
                break
    torch.cuda.synchronize()
    for a, b in pending:
        total += a.elapsed_time(b)
    return {"launches": n, "ms": round(total, 1)}


def time_calls(call, stream, steps):
    """Device time of `call` on `stream`. The timed region is `steps` back-to-back calls
    between one pair of HIP events recorded on that stream: its length / steps is the
    average. A second pass brackets every call with its own events for the median and
    minimum; an event between calls leaves a gap of a few microseconds, so that pass
    does not give the average."""
    import torch

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    total_ms = t0.elapsed_time(t1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    return dict(avg=total_ms / steps, total=total_ms, median=per[len(per) // 2], min=per[0],
                wall_ms=(wall1 - wall0) * 1e3)


def time_workload(w, steps, warmup, settle_ms=SETTLE_MS):
    import torch
    import exact_attention_forward_fwd_amd as fa
    from exact_attention_forward_fwd_amd.workloads import make_inputs

    dev = torch.device("cuda:0")
    q, k, v, _ = make_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    tile = w.tile or (None, None)
    # One call through the checked binding; the timed calls then go straight to the C
    # entry point with the arguments marshalled once. The binding's per-call checks cost
    # the host tens of microseconds, more than a short kernel (about 30 us at N = 1000):
    # back to back, the GPU would then idle between launches.
    fa.fwd(q, k, v, scale=w.scale, causal=w.causal, block_m=tile[0], block_n=tile[1],
           out=o, lse=lse, stream=stream)
    from exact_attention_forward_fwd_amd import _binding
    lib = _binding.load_library()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H, w.N, w.d,
            float(w.scale), int(w.causal), _binding._dtype_code(q), stream.cuda_stream)
    if w.tile:
        args = args + tuple(w.tile)
    entry = lib.fa_fwd_tiled if w.tile else lib.fa_fwd

    def step():
        st = entry(*args)
        if st != 0:
            raise _binding.FaError(st, "fa_fwd")

    sett = settle(step, stream, settle_ms, steps)
    for _ in range(warmup):
        step()
    # one launch per step: the step time is the kernel's average launch duration
    t = time_calls(step, stream, steps)
    return dict(ms_per_step=t["avg"], kernel_ms_avg=t["avg"], kernel_ms_median=t["median"],
                kernel_ms_min=t["min"], wall_ms_per_step=t["wall_ms"] / steps, settle=sett, inputs=(q, k, v))


def time_split(w, steps, warmup, settle_ms=SETTLE_MS):
    """Per-call device time of fa_fwd_split (attention launch + merge launch) at the
    library's suggested split count, and of the unsplit call, on the same inputs: five
    alternating rounds of steps / 5 back-to-back calls each; call_ms_median is the
    median round."""
    import torch
    import exact_attention_forward_fwd_amd as fa
    from exact_attention_forward_fwd_amd.workloads import make_general_inputs

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_general_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    dt = fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16
    splits = fa.fa_split_default(w.B, w.Hq, w.Hk, w.Nq, w.Nk, w.d, w.causal)
    ws_bytes = fa.fa_split_workspace_bytes(w.B, w.Hq, w.Nq, w.d, splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    lib = fa.load_library()
    st = [fa._binding._strides(t.stride()[:3]) for t in (q, k, v, o)]
    base = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.Hq, w.Hk, w.Nq, w.Nk,
            w.d, *st, float(w.scale), int(w.causal), dt, sp, 0, 0)

    def caller(n_splits):
        def call():
            rc = lib.fa_fwd_split(*base, n_splits, ws.data_ptr(), ws.numel())
            if rc != 0:
                raise fa.FaError(rc, "fa_fwd_split")
        return call

    # the split and unsplit calls alternate in rounds, so that both see the same clock
    call_s, call_1 = caller(splits), caller(1)
    settle(call_s, stream, settle_ms, steps)
    for _ in range(warmup):
        call_s()
        call_1()
    rounds = 5
    per = max(1, steps // rounds)
    t_s, t_1 = [], []
    for _ in range(rounds):
        t_s.append(time_calls(call_s, stream, per)["avg"])
        t_1.append(time_calls(call_1, stream, per)["avg"])
    avg, avg1 = sum(t_s) / rounds, sum(t_1) / rounds
    med = sorted(t_s)[rounds // 2]
    rec = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hk": w.Hk, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
           "dtype": w.dtype, "causal": w.causal, "splits": splits,
           "call_ms_avg": round(avg, 5), "call_ms_median": round(med, 5),
           "unsplit_ms_avg": round(avg1, 5), "speedup_vs_unsplit": round(avg1 / avg, 2)}
    if w.flops / w.hbm_bytes < MFMA_PEAK_TFLOPS / (HBM_PEAK_GBS * 1e-3):
        # below the ridge point (decoding): bounded by streaming K and V from HBM
        gbs = w.hbm_bytes / (avg * 1e-3) / 1e9
        rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": w.hbm_bytes}
    else:
        tf = w.flops / (avg * 1e-3) / 1e12
        rec["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / MFMA_PEAK_TFLOPS, 4), "algorithmic_flop": w.flops}
    return rec


def time_backward(w, steps, warmup, settle_ms=SETTLE_MS):
    """Per-call device time of fa_bwd (two launches: the dQ kernel, which also forms the
    row terms D = dO.O and the base-2 LSE, then the dK/dV kernel) on a forward benchmark
    workload with dO ~ N(0, 1), o and lse from fa_fwd. Algorithmic FLOPs are the five
    products of the gradient (S, dP, dV, dK, dQ: 2.5x the forward's); the kernels
    execute seven (S and dP once more in the dQ kernel)."""
    import torch
    import exact_attention_forward_fwd_amd as fa
    from exact_attention_forward_fwd_amd.workloads import make_inputs

    dev = torch.device("cuda:0")
    q, k, v, _ = make_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    g = torch.Generator("cpu").manual_seed(5000 + w.index)
    do = torch.randn(q.shape, generator=g).to(q.dtype).to(dev)
    o, lse = fa.fwd(q, k, v, scale=w.scale, causal=w.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    lib = fa.load_library()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), w.B, w.H, w.N, w.d, float(w.scale), int(w.causal),
            fa.FA_F16 if w.dtype == "f16" else fa.FA_BF16, ws.data_ptr(), ws.numel(), stream.cuda_stream)

    def call():
        rc = lib.fa_bwd(*args)
        if rc != 0:
            raise fa.FaError(rc, "fa_bwd")

    settle(call, stream, settle_ms, steps)
    for _ in range(warmup):
        call()
    t = time_calls(call, stream, steps)
    avg = t["avg"]
    alg = 2.5 * w.flops
    tf = alg / (avg * 1e-3) / 1e12
    return {"workload": w.name, "dtype": w.dtype, "causal": w.causal, "call_ms_avg": round(avg, 5),
            "call_ms_median": round(t["median"], 5),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_PEAK_TFLOPS, 4), "algorithmic_flop": alg,
                         "executed_flop": 3.5 * w.flops}}


def cpu_model() -> str:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_backward(w, budget_s=6.0):
    """The fp64 oracle's backward on whole (b, h) slices of the workload until the budget
    is spent (at least one slice), priced at the same algorithmic FLOPs."""
    import oracle
    from exact_attention_forward_fwd_amd.workloads import make_inputs

    q, k, v, _ = make_inputs(w)
    q = q.double().numpy().reshape(-1, w.N, w.d)
    k = k.double().numpy().reshape(-1, w.N, w.d)
    v = v.double().numpy().reshape(-1, w.N, w.d)
    import numpy as np
    do = np.random.default_rng(5000 + w.index).standard_normal(q.shape)
    slices = 0
    t0 = time.perf_counter()
    while slices < q.shape[0]:
        n = min(16, q.shape[0] - slices)   # one slice per thread
        oracle.attention_bwd(q[slices:slices + n], k[slices:slices + n], v[slices:slices + n],
                             do[slices:slices + n], w.scale, w.causal)
        slices += n
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    alg = 2.5 * w.flops / (w.B * w.H) * slices
    return {"value": alg / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{slices} of {w.B * w.H} (batch, head) slices of {w.label()}, every gradient, fp64 C "
                      f"oracle backward, {dt:.1f} s"}


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle on this workload's inputs: whole (b, h) slices, in order, until
    the budget is spent (at least one slice)."""
    import numpy as np
    import oracle
    from exact_attention_forward_fwd_amd.workloads import make_inputs

    q, k, v, _ = make_inputs(w)
    q = q.double().numpy(); k = k.double().numpy(); v = v.double().numpy()
    q = q.reshape(-1, w.N, w.d); k = k.reshape(-1, w.N, w.d); v = v.reshape(-1, w.N, w.d)
    slices = 0
    t0 = time.perf_counter()
    # time one slice first to size the sample
    while slices < q.shape[0]:
        oracle.attention_fwd(q[slices], k[slices], v[slices], w.scale, w.causal)
        slices += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = w.flops / (w.B * w.H) * slices
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{slices} of {w.B * w.H} (batch, head) slices of {w.label()}, every row, "
                      f"fp64 three-pass C oracle, {dt:.1f} s"}


def main():
    args = parse()
    if args.traffic_from:
        from exact_attention_forward_fwd_amd.workloads import WORKLOADS
        print(json.dumps(traffic_record(WORKLOADS[args.workload], *args.traffic_from), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X and has no "
              "multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import exact_attention_forward_fwd_amd as fa
    from exact_attention_forward_fwd_amd.workloads import WORKLOADS

    fa.load_library()
    w = WORKLOADS[args.workload]
    if args.profile:
        profile_mode(w, backward=args.backward)
        return
    r = time_workload(w, args.steps, args.warmup, args.settle_ms)
    tflops = w.flops / (r["ms_per_step"] * 1e-3) / 1e12
    achieved = w.flops / (r["kernel_ms_avg"] * 1e-3) / 1e12
    rec = stored_traffic(w)
    traffic = round(rec["hbm_bytes_per_launch"]) if rec else None
    alg_bytes = algorithmic_bytes(w)
    out = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d, halved for causal) and % of MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"min_device_ms": args.settle_ms, "launches": r["settle"]["launches"],
                   "device_ms": r["settle"]["ms"]},
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q, K, V; no dataset)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.scale, "tile": list(w.tile) if w.tile else None,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100 * tflops / MFMA_PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": alg_bytes,
                     "algorithmic_flop": w.flops,
                     "kernel_ms_avg": round(r["kernel_ms_avg"], 5),
                     "kernel_ms_median": round(r["kernel_ms_median"], 5),
                     "hbm_gbs_algorithmic": round(alg_bytes / (r["kernel_ms_avg"] * 1e-3) / 1e9, 1)},
    }
    del r
    if not args.no_others:
        others = []
        for idx in sorted(WORKLOADS):
            if idx == w.index:
                continue
            wo = WORKLOADS[idx]
            # as many timed steps as the headline: a timed region of a few short launches
            # (10 x 30 us) is stretched by the launch latency after its opening synchronisation
            ro = time_workload(wo, args.steps, args.warmup, args.settle_ms)
            tf = wo.flops / (ro["kernel_ms_avg"] * 1e-3) / 1e12
            others.append({"workload": wo.name, "dtype": wo.dtype, "causal": wo.causal,
                           "kernel_ms_avg": round(ro["kernel_ms_avg"], 5),
                           "tflops": round(tf, 2), "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS, 4)})
            del ro
            torch.cuda.empty_cache()
        out["other_workloads"] = others
        from exact_attention_forward_fwd_amd.workloads import SPLIT_WORKLOADS
        out["split_kv"] = [time_split(ws, args.steps, args.warmup, args.settle_ms)
                           for ws in SPLIT_WORKLOADS.values()]
        torch.cuda.empty_cache()
        out["backward"] = [time_backward(WORKLOADS[i], args.steps, args.warmup, args.settle_ms)
                           for i in (2, 4, 3)]
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            out["backward"][0]["cpu_baseline"] = cpu_baseline_backward(WORKLOADS[2])
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
