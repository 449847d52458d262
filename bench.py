#!/usr/bin/env python
"""Benchmark of the dynamic short convolution hot path on one MI355X.

One step = the whole hot path over one synthetic batch of 16,384 tokens
through the two dynamic-conv layers of a ~2B-parameter block:
  MLP intermediate, head-wise  (B=4 T=4096 D=8192 W=4, H=16: 512 filters per
                                token, residual)           forward + backward,
  QKV, low-rank, packed seqs   (B=4 T=4096 D=6144 W=4, R=64: filters generated
                                on chip; sequences of 256..4096 tokens)
                                                           forward + backward,
all through the C ABI of libdsc.so with inputs resident in HBM.

Prints one JSON line: tokens/s of the step (wall time of K steps bracketed by
device synchronisation), achieved algorithmic HBM GB/s, per-entry-point
figures (each call timed with HIP events on the stream it runs on, after a
1 GiB read that evicts the last-level cache, median / min / mean over at
least 50 calls), the roofline of the dominant entry point, the streaming
ceiling measured with the library's own streaming kernel, and, as extras, the
QKV ~150M step (head-wise H=64 and low-rank R=32 at B=8 T=2048 D=2304), the
static short convolution beside the dynamic head-wise layer, decoding steps,
the head-wise and low-rank layers fused with the rotary embedding, the
head-wise layer with filters generated on chip from a hidden state, the fixed-order
backward passes, and the fp64 CPU oracle timed on a bounded sample of the
step's work.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E
METRIC = "dynamic-conv fwd+bwd tokens/s and achieved HBM GB/s (% of peak), 1 MI355X"


def algorithmic_bytes(kind: str, direction: str, B, T, D, W, H=1, R=0, es=2) -> int:
    """Each input read once, each output written once (the low-rank filters are never stored)."""
    N = B * T
    act = N * D * es
    if kind == "static":  # one (D, W) filter, read once; dc is fp32
        return 2 * act + D * W * es if direction == "fwd" else 3 * act + D * W * es + D * W * 4
    if kind == "headwise":
        filt = N * (D // H) * W * es
        return 2 * act + filt if direction == "fwd" else 3 * act + 2 * filt
    zb, ub = N * R * es, R * D * W * es
    if direction == "fwd":
        return 2 * act + zb + ub
    return 3 * act + 2 * zb + ub + R * D * W * 4  # dU is fp32


class Case:
    """Device tensors and the two entry-point calls of one workload."""

    def __init__(self, wl, torch, binding, inputs):
        self.wl = wl
        inp = inputs.make_inputs(wl)
        dev = "cuda"
        self.x, self.dy = inp["x"].to(dev), inp["dy"].to(dev)
        self.cu = None if inp["cu_seqlens"] is None else torch.from_numpy(inp["cu_seqlens"]).to(dev)
        self.y, self.dx = torch.empty_like(self.x), torch.empty_like(self.x)
        self.b = binding
        if wl.kind == "headwise":
            self.w = inp["w"].to(dev)
            self.dw = torch.empty_like(self.w)
        elif wl.kind == "static":
            self.c = inp["c"].to(dev)
            self.dc = torch.empty(self.c.shape, dtype=torch.float32, device=dev)
        else:
            self.z, self.U = inp["z"].to(dev), inp["U"].to(dev)
            self.dz = torch.empty_like(self.z)
            self.dU = torch.empty(self.U.shape, dtype=torch.float32, device=dev)
            nws = binding.dsc_lowrank_bwd_workspace_size(self.x.dtype, wl.B, wl.T, wl.D, wl.W, wl.R)
            self.ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)

    def fwd(self):
        wl = self.wl
        if wl.kind == "headwise":
            self.b.dsc_headwise_fwd(self.x, self.w, self.y, cu_seqlens=self.cu, residual=wl.residual)
        elif wl.kind == "static":
            self.b.dsc_static_fwd(self.x, self.c, self.y, cu_seqlens=self.cu, residual=wl.residual)
        else:
            self.b.dsc_lowrank_fwd(self.x, self.z, self.U, self.y, W=wl.W, cu_seqlens=self.cu,
                                   residual=wl.residual)

    def bwd(self):
        wl = self.wl
        if wl.kind == "headwise":
            self.b.dsc_headwise_bwd(self.x, self.w, self.dy, self.dx, self.dw, cu_seqlens=self.cu,
                                    residual=wl.residual)
        elif wl.kind == "static":
            self.b.dsc_static_bwd(self.x, self.c, self.dy, self.dx, self.dc, cu_seqlens=self.cu,
                                  residual=wl.residual)
        else:
            self.b.dsc_lowrank_bwd(self.x, self.z, self.U, self.dy, self.dx, self.dz, self.dU, self.ws,
                                   W=wl.W, cu_seqlens=self.cu, residual=wl.residual)

    def bytes(self, direction):
        wl = self.wl
        return algorithmic_bytes(wl.kind, direction, wl.B, wl.T, wl.D, wl.W, wl.H, wl.R)

    def flops(self, direction):
        wl = self.wl
        nd = wl.N * wl.D
        if wl.kind in ("headwise", "static"):
            return (2 if direction == "fwd" else 4) * wl.W * nd
        return (2 * wl.R * wl.W + 2 * wl.W) * nd * (1 if direction == "fwd" else 3)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "input_dependent_short_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(entry: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("entries", {}).get(entry, {}).get("bytes_per_launch")


def cpu_baseline(wls, seconds: float):
    """fp64 oracle on the first S tokens of the step's workloads (both layers,
    forward + backward; packed sequences cut at the sample's end), S grown
    until about `seconds` of CPU work."""
    import numpy as np

    import oracle
    from input_dependent_short_amd import inputs
    from input_dependent_short_amd.inputs import to_f64

    full = {wl.kind: inputs.make_inputs(wl) for wl in wls}
    T = min(wl.T for wl in wls)
    Bmax = min(wl.B for wl in wls)

    def sample(d, S):
        # S <= T: the first S tokens of row 0; beyond that whole rows
        out = {}
        for n, v in d.items():
            if n == "cu_seqlens":
                if v is not None:
                    cu = [int(c) for c in v if c < S]
                    out[n] = np.array(cu + [S], dtype=np.int32)
                else:
                    out[n] = None
            elif n == "U":
                out[n] = to_f64(v)
            elif S <= T:
                out[n] = to_f64(v[0:1, :S])
            else:
                out[n] = to_f64(v[0:S // T])
        return out

    def run(S):
        a = {wl.kind: sample(full[wl.kind], S) for wl in wls}
        t0 = time.perf_counter()
        for wl in wls:
            sl = a[wl.kind]
            kw = dict(residual=wl.residual, cu_seqlens=sl["cu_seqlens"])
            if wl.kind == "headwise":
                oracle.headwise_fwd(sl["x"], sl["w"], **kw)
                oracle.headwise_bwd(sl["x"], sl["w"], sl["dy"], **kw)
            else:
                oracle.lowrank_fwd(sl["x"], sl["z"], sl["U"], wl.W, **kw)
                oracle.lowrank_bwd(sl["x"], sl["z"], sl["U"], sl["dy"], wl.W, **kw)
        return time.perf_counter() - t0

    def clamp(S):
        S = max(64, min(S, Bmax * T))
        return S if S <= T else (S // T) * T

    S = 64
    t = run(S)
    while t < seconds / 8 and S < Bmax * T:
        S = clamp(S * 4)
        t = run(S)
    if t < seconds * 0.7 and S < Bmax * T:
        S = clamp(int(S * seconds / max(t, 1e-3)))
        t = run(S)
    passes = 1
    while t < seconds * 0.8 and passes < 64:  # the whole batch is the sample: repeat it
        t += run(S)
        passes += 1
    desc = f"first {S} tokens of row 0" if S <= T else f"first {S // T} rows ({S} tokens)"
    if passes > 1:
        desc += f", {passes} passes"
    return {"value": passes * S / t, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{desc} of the step's batch through both layers ({', '.join(wl.name for wl in wls)}), "
                      f"forward + backward in fp64; {t:.1f} s of CPU time",
            "host": platform.processor() or platform.machine()}


COPY_BYTES = 1 << 30  # bytes read (and written) by the copy-kernel reference


def copy_rate(torch, nbytes: int, flush, reps: int = 20) -> float:
    """GB/s of one device copy (the runtime's) that moves `nbytes` in all
    (half read, half written), timed per launch like the entry points: the
    streaming rate a single kernel of that size reaches, ramp and tail
    included, each copy after a cache flush."""
    half = nbytes // 2
    src = torch.empty(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        flush()
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    t = ts[len(ts) // 2] * 1e-3
    del src, dst
    torch.cuda.empty_cache()
    return 2 * half / t / 1e9


def copy_ceiling(torch, reps: int = 10) -> float:
    """GB/s of a plain device copy (1 GiB read + 1 GiB written): the practical
    streaming ceiling beside the nominal 8 TB/s, and the reference kernel of
    known size that scales the HBM byte counters."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / t / 1e9


# kernels launched by each entry point (rocprofv3 kernel names contain these)
# entry point -> (main kernels, helper kernels launched by the same call)
ENTRY_KERNELS = {
    "dsc_headwise_fwd": (["hw_fwd_kernel"], []),
    "dsc_headwise_bwd": (["hw_bwd_kernel"], []),
    "dsc_lowrank_fwd": (["lr_fwd_wide", "lr_fwd_mfma", "lr_fwd_generic"], []),
    "dsc_lowrank_bwd": (["lr_bwd_taps", "lr_bwd_mfma", "lr_bwd_generic"], ["clear2", "fill_zero_f32", "cast_f32_bf16"]),
    "dsc_static_fwd": (["st_fwd_kernel"], []),
    "dsc_static_bwd": (["st_bwd_kernel"], ["st_zero"]),
    "dsc_headwise_decode": (["hw_decode_kernel"], []),
    "dsc_lowrank_decode": (["lr_decode_kernel"], []),
    "dsc_rope_table": (["rope_table_kernel"], []),
}


def _counter_rows(d: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_counters(fetch_dir: str, write_dir: str, out_json: str) -> dict:
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch, from two rocprofv3
    --pmc runs of this script) per entry point, scaled by what the same
    counters read for the 1 GiB copy kernel; written to profiles/traffic.json."""
    per = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for r in _counter_rows(d):
            if r.get("Counter_Name") != name:
                continue
            k = r["Kernel_Name"]
            e = per.setdefault(k, {}).setdefault(name, [])
            e.append(float(r["Counter_Value"]))
    copy_k = [k for k in per if "copy" in k.lower()]
    copy_k = max(copy_k, key=lambda k: max(per[k].get("FETCH_SIZE", [0])))
    cf = per[copy_k]

    def largest(vals):  # dispatches of the 1 GiB reference copy (other copies are smaller)
        top = max(vals)
        big = [v for v in vals if v >= 0.5 * top]
        return sum(big) / len(big)

    f_fetch = COPY_BYTES / (largest(cf["FETCH_SIZE"]) * 1024.0)
    f_write = COPY_BYTES / (largest(cf["WRITE_SIZE"]) * 1024.0)
    entries = {}
    for entry, (mains, helpers) in ENTRY_KERNELS.items():
        main_k = [k for k in per if any(pt in k for pt in mains)]
        if not main_k:
            continue
        calls = sum(len(per[k].get("FETCH_SIZE", [])) for k in main_k)
        fetch = write = 0.0
        for k in per:
            if any(pt in k for pt in mains + helpers):
                fetch += sum(per[k].get("FETCH_SIZE", [])) * 1024.0 * f_fetch
                write += sum(per[k].get("WRITE_SIZE", [])) * 1024.0 * f_write
        entries[entry] = {"fetch_bytes_per_launch": fetch / calls, "write_bytes_per_launch": write / calls,
                          "bytes_per_launch": (fetch + write) / calls, "launches": calls}
    rec = {"kernel_source_hash": kernel_source_hash(), "copy_kernel": copy_k,
           "fetch_scale": f_fetch, "write_scale": f_write, "entries": entries}
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def log(msg: str) -> None:
    """Progress line on stderr (the JSON result is the only line on stdout)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


class Flush:
    """Evicts the caches before a timed call: the library's streaming kernel
    reads a 1 GiB buffer with the default cache policy, which replaces the
    256 MB last-level cache and the 4 MB L2 of each XCD with clean lines (a
    write would leave dirty lines whose write-back then runs during the timed
    call)."""

    def __init__(self, torch, binding, nbytes=1 << 30):
        self.buf = torch.full((nbytes,), 1, dtype=torch.uint8, device="cuda")
        self.sink = torch.empty(16, dtype=torch.uint8, device="cuda")
        self.binding = binding
        self.n = nbytes

    def __call__(self):
        self.binding.dsc_bench_stream(self.buf, self.n, self.sink, 0, unroll=8)


def timed_calls(torch, calls, iters, flush):
    """Each call of `calls` (name -> fn) timed `iters` times with HIP events on
    the current stream, each after a cache flush; returns name -> sorted list
    of milliseconds."""
    evs = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(iters)] for k in calls}
    torch.cuda.synchronize()
    for it in range(iters):
        for k, fn in calls.items():
            flush()
            a, b = evs[k][it]
            a.record()
            fn()
            b.record()
    torch.cuda.synchronize()
    return {k: sorted(a.elapsed_time(b) for a, b in v) for k, v in evs.items()}


def entry_figures(ms, nbytes, flops, entry, workload):
    avg = sum(ms) / len(ms)
    med, mn = ms[len(ms) // 2], ms[0]
    return {"entry": entry, "workload": workload, "calls": len(ms), "avg_us": round(avg * 1e3, 2),
            "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (avg * 1e-3) / 1e9, 1),
            "GBps_median": round(nbytes / (med * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "TFLOPs": round(flops / (avg * 1e-3) / 1e12, 2)}


ENTRY = {"headwise_fwd": "dsc_headwise_fwd", "headwise_bwd": "dsc_headwise_bwd",
         "lowrank_fwd": "dsc_lowrank_fwd", "lowrank_bwd": "dsc_lowrank_bwd"}


def step_calls(cases):
    return {f"{c.wl.kind}_{d}": (c, d) for c in cases for d in ("fwd", "bwd")}


def measure_step(torch, cases, K, warmup, iters, flush):
    """Wall time of K steps (nothing but the entry-point calls inside), then
    every call of the step timed on its own after a cache flush."""
    calls = step_calls(cases)

    def step():
        for c, d in calls.values():
            (c.fwd if d == "fwd" else c.bwd)()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = timed_calls(torch, {k: (c.fwd if d == "fwd" else c.bwd) for k, (c, d) in calls.items()}, iters, flush)
    per = {k: entry_figures(ms[k], c.bytes(d), c.flops(d), ENTRY[k], c.wl.name) for k, (c, d) in calls.items()}
    # each layer's forward + backward back to back, K times, wall clock: the
    # rate a training step sees (each call's writes are paid by the calls
    # after it, as in a real step)
    pairs = {}
    for c in cases:
        for _ in range(2):
            c.fwd(); c.bwd()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            c.fwd(); c.bwd()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / K * 1e6
        b = c.bytes("fwd") + c.bytes("bwd")
        pairs[c.wl.name] = {"fwd_bwd_step_us": round(us, 1), "tokens_per_s": round(c.wl.N / (us * 1e-6), 1),
                            "GBps": round(b / (us * 1e-6) / 1e9, 1),
                            "frac_hbm_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
    return wall / K * 1e3, per, pairs


def interleaved_s(torch, calls, reps):
    """Seconds per call of each of `calls`, run in turn in one loop (after 3
    untimed rounds), from events between consecutive calls."""
    for _ in range(3):
        for f in calls:
            f()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(reps)]
    for e in evs:
        e[0].record()
        for i, f in enumerate(calls):
            f()
            e[i + 1].record()
    torch.cuda.synchronize()
    return [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / reps * 1e-3 for i in range(len(calls))]


def steady_us(torch, fn, reps):
    """Microseconds per call of `fn` launched `reps` times back to back
    (HIP events around the batch): the steady state, where every call also
    pays for the write-back of the lines its predecessors left dirty."""
    for _ in range(2):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def stream_ceiling(torch, binding, mixes, reps):
    """Best steady-state rate of the library's streaming kernel
    (dsc_bench_stream) over a few recipes, for each read / write byte mix:
    the practical ceiling of a kernel that moves those bytes."""
    top = max(max(r, w) for r, w in mixes.values())
    src = torch.empty(top, dtype=torch.uint8, device="cuda")
    dst = torch.empty(top, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    recipes = [dict(unroll=u, load_nt=ln, store_nt=sn, chunked=False, blocks=bl) for u in (1, 4)
               for ln in (False, True) for sn in (False, True) for bl in (0, 4 * cus)]
    out = {}
    for name, (rb, wb) in mixes.items():
        best = None
        for rcp in recipes:
            us = steady_us(torch, lambda rb=rb, wb=wb, rcp=rcp: binding.dsc_bench_stream(src, rb, dst, wb, **rcp), reps)
            gbps = (rb + wb) / (us * 1e-6) / 1e9
            if best is None or gbps > best[0]:
                best = (gbps, rcp, us)
        gbps, rcp, us = best
        out[name] = {"read_bytes": rb, "write_bytes": wb, "GBps": round(gbps, 1), "us": round(us, 2),
                     "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4), "recipe": rcp}
    del src, dst
    torch.cuda.empty_cache()
    return out


def stream_sweep(torch, binding, inputs) -> int:
    """Every recipe of dsc_bench_stream on the byte mixes of the MLP ~2B
    head-wise layer (a 268 MB activation, its forward and backward mixes, pure
    reads and writes, and a 1 GiB copy), each timed in steady state; prints
    the best and worst recipes of each mix."""
    wl = inputs.WORKLOADS[4]
    act = wl.N * wl.D * 2
    filt = wl.N * (wl.D // wl.H) * wl.W * 2
    mixes = {"copy_activation": (act, act), "copy_1GiB": (1 << 30, 1 << 30),
             "headwise_fwd_mix": (act + filt, act), "headwise_bwd_mix": (2 * act + filt, act + filt),
             "read_only": (3 * act + filt, 0), "write_only": (0, act + filt)}
    top = max(max(r, w) for r, w in mixes.values())
    src = torch.full((top,), 3, dtype=torch.uint8, device="cuda")
    dst = torch.empty(top, dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for name, (rb, wb) in mixes.items():
        rows = []
        for u in (1, 2, 4, 8):
            for lnt, snt in ((False, False), (True, False), (False, True), (True, True)):
                for ch in (False, True):
                    for bl in (0, cus * 2, cus * 4, cus * 16, cus * 64):
                        rcp = dict(unroll=u, load_nt=lnt, store_nt=snt, chunked=ch, blocks=bl)
                        us = steady_us(torch, lambda rcp=rcp: binding.dsc_bench_stream(src, rb, dst, wb, **rcp), 10)
                        rows.append((round((rb + wb) / (us * 1e-6) / 1e9, 1), rcp))
        rows.sort(key=lambda r: -r[0])
        log(f"sweep {name}: best {rows[0]}")
        print(json.dumps({"mix": name, "read_bytes": rb, "write_bytes": wb, "best": rows[:8],
                          "worst": rows[-3:], "n": len(rows)}), flush=True)
    return 0


def summarize_sq(dirs, kernels=("hw_fwd_kernel", "hw_bwd_kernel", "lr_fwd_wide", "lr_fwd_mfma", "lr_bwd_mfma",
                                 "lr_bwd_taps", "lr_dz_", "lr_bwd_generic", "st_fwd_kernel", "st_bwd_kernel")) -> str:
    """Markdown table of the SQ counters (rocprofv3 --pmc passes of this
    script, one directory each) of the convolution kernels, averaged per
    dispatch: instructions per wave, vector-ALU and matrix-core busy fractions
    per SIMD, LDS bank conflicts per active LDS cycle."""
    import collections
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for r in _counter_rows(d):
            k = r["Kernel_Name"]
            if any(p in k for p in kernels):
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                vals[k]["VGPR"] = [float(r["VGPR_Count"])]
                vals[k]["AGPR"] = [float(r.get("Accum_VGPR_Count") or 0)]
    avg = lambda k, c: (sum(vals[k][c]) / len(vals[k][c])) if vals[k].get(c) else float("nan")
    out = ["| kernel | waves | VGPR + AGPR | VALU / wave | MFMA / wave | LDS / wave | SALU / wave | "
           "VMEM rd / wave | VMEM wr / wave | VALU busy | matrix cores busy | waiting / wave cycles | "
           "LDS conflict / LDS active |", "|" + "---|" * 13]
    for k in sorted(vals):
        w = avg(k, "SQ_WAVES")
        cyc = avg(k, "GRBM_GUI_ACTIVE") / 8.0  # the counter sums the 8 XCDs
        simds = 1024.0
        name = k.replace("void ", "").replace("dsc::(anonymous namespace)::", "").replace("dsc::", "")
        name = name[:name.index(">") + 1] if ">" in name else name.split("(")[0]
        out.append(f"| `{name}` | {w:.0f} | {avg(k, 'VGPR'):.0f} + {avg(k, 'AGPR'):.0f} | "
                   f"{avg(k, 'SQ_INSTS_VALU') / w:.0f} | {avg(k, 'SQ_INSTS_MFMA') / w:.0f} | "
                   f"{avg(k, 'SQ_INSTS_LDS') / w:.0f} | {avg(k, 'SQ_INSTS_SALU') / w:.0f} | "
                   f"{avg(k, 'SQ_INSTS_VMEM_RD') / w:.0f} | {avg(k, 'SQ_INSTS_VMEM_WR') / w:.0f} | "
                   f"{avg(k, 'SQ_ACTIVE_INST_VALU') * 4 / simds / cyc:.0%} | "
                   f"{avg(k, 'SQ_VALU_MFMA_BUSY_CYCLES') / simds / cyc:.0%} | "
                   f"{avg(k, 'SQ_WAIT_INST_ANY') / max(avg(k, 'SQ_WAVE_CYCLES'), 1):.0%} | "
                   f"{avg(k, 'SQ_LDS_BANK_CONFLICT') / max(avg(k, 'SQ_ACTIVE_INST_LDS'), 1):.2f} |")
    return "\n".join(out)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--iters", type=int, default=50,
                    help="flushed calls timed per entry point (the default run uses at least 50; fewer only with "
                         "--headline-only, for profiler passes)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the 2B step and its copy reference (for counter runs: every launch of an "
                         "entry point's kernels then belongs to the headline workload)")
    ap.add_argument("--no-deterministic", action="store_true",
                    help="skip the timing of the fixed-order backward passes (whose kernel launches would "
                         "otherwise mix with the fast backward's in a kernel trace)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of this script into profiles/traffic.json")
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR",
                    help="print a markdown table of the SQ counters from rocprofv3 --pmc passes of this script")
    ap.add_argument("--stream-sweep", action="store_true",
                    help="only sweep the streaming kernel's recipes (loads in flight, cache policies, order, "
                         "grid size) over the byte mixes of the 2B head-wise layer; one JSON line per mix")
    args = ap.parse_args()

    if args.summarize_sq:
        print(summarize_sq(args.summarize_sq))
        return 0
    if args.summarize_counters:
        rec = summarize_counters(*args.summarize_counters, os.path.join(ROOT, "profiles", "traffic.json"))
        print(json.dumps(rec, indent=1))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the dynamic short convolution is per-token local and this build runs on a single "
              "MI355X.", file=sys.stderr)
        return 2

    import torch

    from input_dependent_short_amd import binding, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    binding.lib()  # fails loudly if the HIP library is not built
    iters = args.iters if args.headline_only else max(50, args.iters)
    if args.stream_sweep:
        return stream_sweep(torch, binding, inputs)
    # a 1 GiB read before every timed call evicts the inputs from the
    # 256 MB last-level cache and the 4 MB L2 of each XCD
    flush = Flush(torch, binding)

    log("copy reference")
    copy_gbps = copy_ceiling(torch)
    log("inputs of the 2B step")
    cases = [Case(inputs.WORKLOADS[4], torch, binding, inputs), Case(inputs.WORKLOADS[5], torch, binding, inputs)]
    K = args.steps
    log("timing the 2B step")
    ms_step, per_call, pairs = measure_step(torch, cases, K, args.warmup, iters, flush)
    N = cases[0].wl.N
    step_bytes = sum(c.bytes(d) for c, d in step_calls(cases).values())
    dom_key = max(per_call, key=lambda k: per_call[k]["avg_us"])
    dom = per_call[dom_key]
    traffic = measured_traffic(dom["entry"])
    hw4, lr5 = cases[0].wl, cases[1].wl

    out = {
        "metric": METRIC,
        "value": round(N / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one batch of 16384 tokens through the two dynamic-conv layers of a ~2B block: "
                               "MLP intermediate head-wise (H=16, residual) and QKV low-rank (R=64, packed "
                               "sequences of 256..4096 tokens), forward+backward",
                   "mlp_headwise": {"B": hw4.B, "T": hw4.T, "D": hw4.D, "W": hw4.W, "H": hw4.H},
                   "qkv_lowrank": {"B": lr5.B, "T": lr5.T, "D": lr5.D, "W": lr5.W, "R": lr5.R,
                                   "sequences": int(len(cases[1].cu) - 1)},
                   "dtype": "bf16"},
        "achieved_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": dom["entry"], "workload": dom["workload"],
                     "achieved": dom["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": dom["frac_hbm_peak"],
                     "traffic": traffic, "bytes_per_launch": dom["algorithmic_bytes"],
                     "avg_launch_us": dom["avg_us"], "median_launch_us": dom["median_us"],
                     "min_launch_us": dom["min_us"]},
        "per_entry": per_call,
        # per layer: forward + backward back to back (wall clock), the rate set
        # against 70% of the 8 TB/s peak
        "fwd_bwd": pairs,
        "copy_ceiling_GBps": round(copy_gbps, 1),
    }
    if args.headline_only:
        print(json.dumps(out), flush=True)
        return 0

    # the practical ceiling of the same byte mixes (and of a plain copy) with
    # the library's own streaming kernel, and of one device copy of the
    # dominant entry's bytes
    log("streaming ceiling")
    c4 = cases[0]
    out["stream_ceiling"] = stream_ceiling(torch, binding, {
        "copy_activation": (c4.x.numel() * 2, c4.x.numel() * 2),
        "headwise_fwd_mix": (c4.bytes("fwd") - c4.x.numel() * 2, c4.x.numel() * 2),
        "headwise_bwd_mix": (c4.bytes("bwd") - c4.x.numel() * 2 - c4.w.numel() * 2,
                             c4.x.numel() * 2 + c4.w.numel() * 2),
        "read_only": (c4.bytes("bwd"), 0),
        "write_only": (0, c4.x.numel() * 2)}, 10)
    out["copy_same_bytes_GBps"] = round(copy_rate(torch, dom["algorithmic_bytes"], flush), 1)

    # the low-rank layer of the ~2B block followed by the rotary embedding of
    # its query and key channels ([0, 4096), heads of 128), forward and
    # backward, beside the layer alone, in one loop
    log("fused rotary embedding, ~2B low-rank")
    l5 = cases[1]
    hd2, rot2 = 128, 4096
    table2 = torch.empty(l5.wl.N, hd2 // 2, 2, dtype=torch.float32, device="cuda")
    binding.dsc_rope_table(table2, base=10000.0)
    lkw2 = dict(W=l5.wl.W, rot=rot2, head_dim=hd2, table=table2, cu_seqlens=l5.cu, residual=l5.wl.residual)
    tr2 = interleaved_s(torch, [
        lambda: binding.dsc_lowrank_rope_fwd(l5.x, l5.z, l5.U, l5.y, **lkw2),
        lambda: binding.dsc_lowrank_rope_bwd(l5.x, l5.z, l5.U, l5.dy, l5.dx, l5.dz, l5.dU, l5.ws, **lkw2),
        l5.fwd, l5.bwd], max(5, K // 2))
    b2 = l5.bytes("fwd") + l5.bytes("bwd")
    rope2b = {"workload": f"{l5.wl.name} + rotary embedding of channels [0, {rot2}), heads of {hd2}",
              "fwd_us": round(tr2[0] * 1e6, 1), "bwd_us": round(tr2[1] * 1e6, 1),
              "GBps": round(b2 / (tr2[0] + tr2[1]) / 1e9, 1),
              "frac_hbm_peak": round(b2 / (tr2[0] + tr2[1]) / 1e9 / PEAK_HBM_GBPS, 4),
              "layer_alone_fwd_us": round(tr2[2] * 1e6, 1), "layer_alone_bwd_us": round(tr2[3] * 1e6, 1),
              "unfused_extra_bytes": 2 * rot2 * l5.wl.N * l5.x.element_size()}
    del cases, c4, l5, table2
    torch.cuda.empty_cache()

    # the QKV ~150M step (head-wise H=64 with residual, low-rank R=32) measured the same way
    log("QKV ~150M step")
    small = [Case(inputs.WORKLOADS[2], torch, binding, inputs), Case(inputs.WORKLOADS[3], torch, binding, inputs)]
    ms_small, per_small, pairs_small = measure_step(torch, small, K, args.warmup, iters, flush)
    small_bytes = sum(c.bytes(d) for c, d in step_calls(small).values())
    out["qkv_150m_step"] = {"workload": "QKV dynamic short conv at ~150M scale: head-wise (H=64, residual) and "
                                        "low-rank (R=32) forward+backward, B=8 T=2048 D=2304 W=4",
                            "ms_per_step": round(ms_small, 4),
                            "tokens_per_s": round(small[0].wl.N / (ms_small * 1e-3), 1),
                            "GBps": round(small_bytes / (ms_small * 1e-3) / 1e9, 1),
                            "fwd_bwd": pairs_small, "per_entry": per_small}
    hwc, lrc = small

    # The pages set the dynamic kernels' latency against optimised kernels of
    # the static short convolution (one fixed filter per channel).  Our own
    # static kernels at the two head-wise shapes, timed the same way (flushed
    # calls), beside the dynamic head-wise figures of this run.
    log("static vs dynamic")
    static = {}
    for cfg, dyn in ((2, (per_small["headwise_fwd"]["avg_us"], per_small["headwise_bwd"]["avg_us"])),
                     (4, (per_call["headwise_fwd"]["avg_us"], per_call["headwise_bwd"]["avg_us"]))):
        hw = inputs.WORKLOADS[cfg]
        wl = inputs.Workload(hw.name.replace("headwise", "static"), "static", hw.B, hw.T, hw.D, hw.W,
                             dtype=hw.dtype, residual=hw.residual, cfg=hw.cfg)
        sc = Case(wl, torch, binding, inputs)
        ms = timed_calls(torch, {"fwd": sc.fwd, "bwd": sc.bwd}, iters, flush)
        tf, tb = (sum(ms[k]) / len(ms[k]) * 1e-3 for k in ("fwd", "bwd"))
        b = sc.bytes("fwd") + sc.bytes("bwd")
        static[wl.name] = {"fwd_us": round(tf * 1e6, 1), "bwd_us": round(tb * 1e6, 1),
                           "GBps": round(b / (tf + tb) / 1e9, 1),
                           "frac_hbm_peak": round(b / (tf + tb) / 1e9 / PEAK_HBM_GBPS, 4),
                           "dynamic_headwise_fwd_us": dyn[0], "dynamic_headwise_bwd_us": dyn[1],
                           "dynamic_over_static": round((dyn[0] + dyn[1]) / ((tf + tb) * 1e6), 3)}
        del sc
        torch.cuda.empty_cache()
    out["static_vs_dynamic"] = static

    # decoding: one new token for each of 64 sequences per step, at the QKV
    # ~150M width (inputs are rows of the step's seeded tensors); the state
    # is updated in place step after step.  us_per_step is a HIP graph of
    # the steps replayed (GPU time); us_per_step_eager launches each step
    # from Python (host-bound at this size)
    log("decoding")
    S_DEC, STEPS_DEC = 64, 200
    D, Wd = hwc.wl.D, hwc.wl.W
    xd = hwc.x.view(-1, D)[:S_DEC].contiguous()
    wd = hwc.w.view(-1, D // hwc.wl.H, Wd)[:S_DEC].contiguous()
    zd = lrc.z.view(-1, lrc.wl.R)[:S_DEC].contiguous()
    yd = torch.empty_like(xd)
    state = torch.zeros(S_DEC, Wd - 1, D, dtype=xd.dtype, device="cuda")
    es = xd.element_size()
    act = S_DEC * D * es
    # the rotated step: queries and keys (channels [0, 1536), heads of 64) at
    # positions 1000 + b, cos / sin rows read once per (sequence, chunk)
    dec_table = torch.empty(2048, 32, 2, dtype=torch.float32, device="cuda")
    binding.dsc_rope_table(dec_table)
    dec_pos = torch.arange(1000, 1000 + S_DEC, dtype=torch.int32, device="cuda")
    dec_calls = {
        "headwise-qkv-150m": (lambda: binding.dsc_headwise_decode(xd, wd, state, yd, residual=True),
                              2 * act + 2 * (Wd - 1) * act + wd.numel() * es),
        "headwise-rope-qkv-150m": (lambda: binding.dsc_headwise_rope_decode(
                                       xd, wd, state, yd, dec_pos, rot=1536, head_dim=64, table=dec_table,
                                       residual=True),
                                   2 * act + 2 * (Wd - 1) * act + wd.numel() * es + S_DEC * 4),
        "lowrank-qkv-150m": (lambda: binding.dsc_lowrank_decode(xd, zd, lrc.U, state, yd, W=Wd),
                             2 * act + 2 * (Wd - 1) * act + zd.numel() * es + lrc.U.numel() * es),
    }
    dec = {}
    for name, (fn, nbytes) in dec_calls.items():
        for _ in range(10):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(STEPS_DEC):
            fn()
        b.record()
        torch.cuda.synchronize()
        t_eager = a.elapsed_time(b) * 1e-3 / STEPS_DEC
        # the same steps captured once as a HIP graph and replayed: the GPU's
        # own time per step, without the host's per-call launch work
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(g):
            for _ in range(STEPS_DEC):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        t = a.elapsed_time(b) * 1e-3 / STEPS_DEC
        dec[name] = {"sequences": S_DEC, "us_per_step": round(t * 1e6, 2),
                     "us_per_step_eager": round(t_eager * 1e6, 2),
                     "tokens_per_s": round(S_DEC / t, 1), "bytes_per_step": nbytes,
                     "GBps": round(nbytes / t / 1e9, 1)}
        del g
    out["decode"] = dec

    # The layer on the query / key / value projections feeds the rotary
    # embedding of the queries and keys.  The fused calls rotate channels
    # [0, 1536) (12 query and 12 key heads of 64) of the QKV ~150M
    # workloads on the fly; the layer alone is timed in the same loop.  A
    # separate rotation pass would move rot*N elements in and out once
    # more in each direction (unfused_extra_bytes per direction).
    log("fused rotary embedding")
    hd, rot = 64, 2 * 768
    table = torch.empty(hwc.wl.T, hd // 2, 2, dtype=torch.float32, device="cuda")
    binding.dsc_rope_table(table, base=10000.0)
    reps = max(5, K // 2)
    rope = {}
    kw = dict(rot=rot, head_dim=hd, table=table, residual=hwc.wl.residual)
    lkw = dict(W=lrc.wl.W, rot=rot, head_dim=hd, table=table, residual=lrc.wl.residual)
    for name, c, calls in (
            ("headwise", hwc, [lambda: binding.dsc_headwise_rope_fwd(hwc.x, hwc.w, hwc.y, **kw),
                               lambda: binding.dsc_headwise_rope_bwd(hwc.x, hwc.w, hwc.dy, hwc.dx, hwc.dw, **kw),
                               hwc.fwd, hwc.bwd]),
            ("lowrank", lrc, [lambda: binding.dsc_lowrank_rope_fwd(lrc.x, lrc.z, lrc.U, lrc.y, **lkw),
                              lambda: binding.dsc_lowrank_rope_bwd(lrc.x, lrc.z, lrc.U, lrc.dy, lrc.dx, lrc.dz,
                                                                   lrc.dU, lrc.ws, **lkw),
                              lrc.fwd, lrc.bwd])):
        tr = interleaved_s(torch, calls, reps)
        b = c.bytes("fwd") + c.bytes("bwd") + 2 * table.numel() * 4
        rope[name] = {
            "workload": f"{c.wl.name} + rotary embedding of channels [0, {rot}), heads of {hd}",
            "fwd_us": round(tr[0] * 1e6, 1), "bwd_us": round(tr[1] * 1e6, 1),
            "GBps": round(b / (tr[0] + tr[1]) / 1e9, 1),
            "frac_hbm_peak": round(b / (tr[0] + tr[1]) / 1e9 / PEAK_HBM_GBPS, 4),
            "layer_alone_fwd_us": round(tr[2] * 1e6, 1), "layer_alone_bwd_us": round(tr[3] * 1e6, 1),
            "unfused_extra_bytes": 2 * rot * c.wl.N * c.x.element_size()}
    rope["lowrank_2b"] = rope2b
    out["rope_fused"] = rope
    del table

    # The head-wise layer with its filters generated from a hidden state of
    # width 2048 (the ~2B block's), at the MLP ~2B shape: the fused calls (w
    # formed on chip, never stored) against the same product written to
    # memory by this library's matrix-core GEMM (dsc_generate_filters), then
    # read by the head-wise layer, and against the ROCm GEMM (torch.matmul) in
    # that role; the backward the same way (library: w, then dx and dw, then
    # dh and dV).  Back to back, in one loop.
    log("generated filters")
    gwl, Kg = inputs.WORKLOADS[4], 2048
    ginp = inputs.generator_inputs(gwl, Kg)
    gx, gdy, gV, gh = (ginp[k].to("cuda") for k in ("x", "dy", "V", "h"))
    del ginp
    Ng, Gg, Wg = gwl.N, gwl.D // gwl.H, gwl.W
    gy, gdx = torch.empty_like(gx), torch.empty_like(gx)
    gdh = torch.empty_like(gh)
    gdV = torch.empty(gV.shape, dtype=torch.float32, device="cuda")
    gw_ = torch.empty(gwl.B, gwl.T, Gg, Wg, dtype=torch.bfloat16, device="cuda")
    gdw = torch.empty_like(gw_)
    gws = torch.empty(binding.dsc_headwise_gen_bwd_workspace_size(gx.dtype, gwl.B, gwl.T, gwl.D, Wg, gwl.H, Kg),
                      dtype=torch.uint8, device="cuda")
    hf, wf, dwf = gh.view(Ng, Kg), gw_.view(Ng, Gg * Wg), gdw.view(Ng, Gg * Wg)
    res = gwl.residual

    def lib_bwd():
        torch.matmul(hf, gV.t(), out=wf)
        binding.dsc_headwise_bwd(gx, gw_, gdy, gdx, gdw, residual=res)
        torch.matmul(dwf, gV, out=gdh.view(Ng, Kg))
        gdV.copy_(torch.matmul(dwf.t(), hf))

    gcalls = {
        "fused_fwd": lambda: binding.dsc_headwise_gen_fwd(gh, gV, gx, gy, W=Wg, residual=res),
        "fused_bwd": lambda: binding.dsc_headwise_gen_bwd(gh, gV, gx, gdy, gdx, gdh, gdV, gws, W=Wg, residual=res),
        "own_gemm_w": lambda: binding.dsc_generate_filters(hf, gV, wf),
        "headwise_fwd": lambda: binding.dsc_headwise_fwd(gx, gw_, gy, residual=res),
        "library_gemm_w": lambda: torch.matmul(hf, gV.t(), out=wf),
        "library_path_bwd": lib_bwd,
    }
    gt = dict(zip(gcalls, interleaved_s(torch, list(gcalls.values()), reps)))
    us = {k: round(v * 1e6, 1) for k, v in gt.items()}
    gflop = 2.0 * Ng * Kg * Gg * Wg
    out["generator_fused"] = {
        "workload": f"{gwl.name} with w = h V^T generated from a hidden state of width {Kg} "
                    f"(B={gwl.B} T={gwl.T} D={gwl.D} W={Wg} H={gwl.H}, V ({Gg * Wg}, {Kg}))",
        "fused_fwd_us": us["fused_fwd"], "fused_bwd_us": us["fused_bwd"],
        "unfused_own_gemm_fwd_us": round(us["own_gemm_w"] + us["headwise_fwd"], 1),
        "unfused_library_gemm_fwd_us": round(us["library_gemm_w"] + us["headwise_fwd"], 1),
        "unfused_library_bwd_us": us["library_path_bwd"],
        "own_gemm_TFLOPs": round(gflop / gt["own_gemm_w"] / 1e12, 1),
        "library_gemm_TFLOPs": round(gflop / gt["library_gemm_w"] / 1e12, 1),
        "w_round_trip_bytes": 2 * Ng * Gg * Wg * 2,
        "per_call_us": us}
    del gx, gdy, gV, gh, gy, gdx, gdh, gdV, gw_, gdw, gws, hf, wf, dwf
    torch.cuda.empty_cache()

    # The reproducible low-rank backward (dz and dU summed in a fixed order
    # through per-block workspace regions) against the fast one, at the
    # QKV ~150M low-rank size, alternating in the same loop.
    if not args.no_deterministic:
        log("fixed-order backward passes")
        lw = lrc.wl
        nws = binding.dsc_lowrank_bwd_deterministic_workspace_size(lrc.x.dtype, lw.B, lw.T, lw.D, lw.W, lw.R)
        det_ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        calls = [lambda: binding.dsc_lowrank_bwd_deterministic(lrc.x, lrc.z, lrc.U, lrc.dy, lrc.dx, lrc.dz, lrc.dU,
                                                               det_ws if nws else None, W=lw.W,
                                                               cu_seqlens=lrc.cu, residual=lw.residual),
                 lrc.bwd]
        td = interleaved_s(torch, calls, reps)
        out["lowrank_bwd_deterministic"] = {
            "workload": lw.name, "us": round(td[0] * 1e6, 1), "fast_us": round(td[1] * 1e6, 1),
            "workspace_bytes": nws, "algorithmic_GBps": round(lrc.bytes("bwd") / td[0] / 1e9, 1)}
        del det_ws

        # The same for the static layer's dc, at the QKV ~150M head-wise shape.
        hw2 = inputs.WORKLOADS[2]
        swl = inputs.Workload(hw2.name.replace("headwise", "static"), "static", hw2.B, hw2.T, hw2.D, hw2.W,
                              dtype=hw2.dtype, residual=hw2.residual, cfg=hw2.cfg)
        sc = Case(swl, torch, binding, inputs)
        nws = binding.dsc_static_bwd_deterministic_workspace_size(sc.x.dtype, swl.B, swl.T, swl.D, swl.W)
        det_ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        calls = [lambda: binding.dsc_static_bwd_deterministic(sc.x, sc.c, sc.dy, sc.dx, sc.dc, det_ws,
                                                              residual=swl.residual),
                 sc.bwd]
        td = interleaved_s(torch, calls, reps)
        out["static_bwd_deterministic"] = {
            "workload": swl.name, "us": round(td[0] * 1e6, 1), "fast_us": round(td[1] * 1e6, 1),
            "workspace_bytes": nws}
        del det_ws, sc

    if not args.no_cpu_baseline:
        log("CPU oracle sample")
        out["cpu_baseline"] = cpu_baseline([inputs.WORKLOADS[4], inputs.WORKLOADS[5]], args.cpu_seconds)
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
