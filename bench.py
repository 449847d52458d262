#!/usr/bin/env python
"""Benchmark of the dynamic short convolution hot path on one MI355X.

One step = the whole hot path over one synthetic batch of the QKV workload
at ~150M scale (B=8, T=2048, D=2304 = Q,K,V of width 768, W=4, bf16):
  head-wise  (H=64, 36 filters per token, residual)  forward + backward,
  low-rank   (R=32, filters generated on chip)       forward + backward,
all through the C ABI of libdsc.so with inputs resident in HBM.

Prints one JSON line: tokens/s of the step, achieved algorithmic HBM GB/s,
the roofline of the dominant entry point (HIP events around each call on
the stream it runs on), per-entry-point figures, the 2B-scale workloads
(head-wise MLP D=8192 H=16 and low-rank varlen D=6144 R=64) timed the same
way, the static short convolution (one fixed filter per channel) at the two
head-wise shapes beside the dynamic figures, one-token decoding steps for 64
sequences, and the fp64 CPU oracle timed on a bounded sample of the step's
work.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
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
    """fp64 oracle on the first S tokens of row 0 of the step's workloads (both
    variants, forward + backward), S grown until about `seconds` of CPU work."""
    import oracle
    from input_dependent_short_amd import inputs
    from input_dependent_short_amd.inputs import to_f64

    full = {wl.kind: inputs.make_inputs(wl) for wl in wls}
    T = min(wl.T for wl in wls)
    Bmax = min(wl.B for wl in wls)

    def sample(d, S):
        # S <= T: the first S tokens of row 0; beyond that whole rows (sequences)
        out = {}
        for n, v in d.items():
            if n == "cu_seqlens":
                continue
            if n == "U":
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
            if wl.kind == "headwise":
                oracle.headwise_fwd(sl["x"], sl["w"], residual=wl.residual)
                oracle.headwise_bwd(sl["x"], sl["w"], sl["dy"], residual=wl.residual)
            else:
                oracle.lowrank_fwd(sl["x"], sl["z"], sl["U"], wl.W, residual=wl.residual)
                oracle.lowrank_bwd(sl["x"], sl["z"], sl["U"], sl["dy"], wl.W, residual=wl.residual)
        return time.perf_counter() - t0

    def clamp(S):
        S = max(64, min(S, Bmax * T))
        return S if S <= T else (S // T) * T

    S = 256
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
            "sample": f"{desc} of the step's batch, head-wise and low-rank forward + backward "
                      f"in fp64; {t:.1f} s of CPU time",
            "host": platform.processor() or platform.machine()}


COPY_BYTES = 1 << 30  # bytes read (and written) by the copy-kernel reference


def copy_rate(torch, nbytes: int, reps: int = 20) -> float:
    """GB/s of one device copy that moves `nbytes` in all (half read, half
    written), timed per launch like the entry points: the streaming rate a
    single kernel of that size reaches, ramp and tail included.  A 512 MiB
    write before every copy evicts the source from the 256 MB last-level
    cache, which would otherwise serve a copy this small."""
    half = nbytes // 2
    src = torch.empty(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        flush.fill_(1)
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    t = ts[len(ts) // 2] * 1e-3
    del src, dst, flush
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
    "dsc_lowrank_bwd": (["lr_bwd_mfma", "lr_bwd_generic"], ["clear2", "fill_zero_f32", "cast_f32_bf16"]),
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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large", action="store_true", help="skip the 2B-scale workloads")
    ap.add_argument("--no-deterministic", action="store_true",
                    help="skip the timing of the reproducible low-rank backward (whose kernel launches would "
                         "otherwise mix with the fast backward's in a kernel trace)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of this script into profiles/traffic.json")
    args = ap.parse_args()

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

    copy_gbps = copy_ceiling(torch)
    cases = [Case(inputs.WORKLOADS[2], torch, binding, inputs), Case(inputs.WORKLOADS[3], torch, binding, inputs)]
    calls = [(f"{c.wl.kind}_{d}", c, d) for c in cases for d in ("fwd", "bwd")]
    names = {"headwise_fwd": "dsc_headwise_fwd", "headwise_bwd": "dsc_headwise_bwd",
             "lowrank_fwd": "dsc_lowrank_fwd", "lowrank_bwd": "dsc_lowrank_bwd"}

    def step(events=None):
        for i, (_, c, d) in enumerate(calls):
            if events is not None:
                events[i][0].record()
            (c.fwd if d == "fwd" else c.bwd)()
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # timed region 1: K whole steps, nothing but the entry-point calls inside
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # timed region 2: the same K steps with HIP events around every call (on
    # the stream the kernels run on), for the per-entry durations; the event
    # records themselves add host and queue work, so region 1 gives the step time
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
          for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        step(ev[k])
    torch.cuda.synchronize()
    per_call = {}
    for i, (key, c, d) in enumerate(calls):
        ms = sorted(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(K))
        avg = sum(ms) / K
        b = c.bytes(d)
        per_call[key] = {"entry": names[key], "workload": c.wl.name, "avg_us": round(avg * 1e3, 2),
                         "median_us": round(ms[K // 2] * 1e3, 2), "algorithmic_bytes": b,
                         "GBps": round(b / (avg * 1e-3) / 1e9, 1),
                         "frac_hbm_peak": round(b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                         "TFLOPs": round(c.flops(d) / (avg * 1e-3) / 1e12, 2)}
    ms_step = wall / K * 1e3
    N = cases[0].wl.N
    step_bytes = sum(c.bytes(d) for _, c, d in calls)
    dom_key = max(per_call, key=lambda k: per_call[k]["avg_us"])
    dom = per_call[dom_key]
    traffic = measured_traffic(dom["entry"])

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
        "config": {"workload": "QKV dynamic short conv at ~150M scale: head-wise (H=64, residual) and "
                               "low-rank (R=32) forward+backward on one batch",
                   "B": 8, "T": 2048, "D": 2304, "W": 4, "H": 64, "R": 32, "dtype": "bf16"},
        "achieved_GBps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": dom["entry"], "achieved": dom["GBps"],
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": dom["frac_hbm_peak"],
                     "traffic": traffic, "bytes_per_launch": dom["algorithmic_bytes"],
                     "avg_launch_us": dom["avg_us"]},
        "per_entry": per_call,
        "copy_ceiling_GBps": round(copy_gbps, 1),
        # a device copy moving as many bytes as the dominant entry's algorithmic traffic
        "copy_same_bytes_GBps": round(copy_rate(torch, dom["algorithmic_bytes"]), 1),
    }

    def fwd_bwd_times(wl, reps):
        """Average fwd and bwd seconds of one workload, HIP events around each call."""
        c = Case(wl, torch, binding, inputs)
        for _ in range(3):
            c.fwd(); c.bwd()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e in evs:
            e[0].record(); c.fwd(); e[1].record(); c.bwd(); e[2].record()
        torch.cuda.synchronize()
        tf = sum(e[0].elapsed_time(e[1]) for e in evs) / reps * 1e-3
        tb = sum(e[1].elapsed_time(e[2]) for e in evs) / reps * 1e-3
        b = c.bytes("fwd") + c.bytes("bwd")
        del c
        torch.cuda.empty_cache()
        return tf, tb, b

    if not args.no_large:
        large = {}
        for cfg in (4, 5):
            wl = inputs.WORKLOADS[cfg]
            tf, tb, b = fwd_bwd_times(wl, max(5, K // 2))
            large[wl.name] = {"tokens_per_s": round(wl.N / (tf + tb), 1),
                              "fwd_us": round(tf * 1e6, 1), "bwd_us": round(tb * 1e6, 1),
                              "GBps": round(b / (tf + tb) / 1e9, 1),
                              "frac_hbm_peak": round(b / (tf + tb) / 1e9 / PEAK_HBM_GBPS, 4)}
        out["workloads_2b"] = large

        # The pages set the dynamic kernels' latency against optimised kernels of
        # the static short convolution (one fixed filter per channel).  Our own
        # static kernels at the two head-wise shapes, timed the same way, beside
        # the dynamic head-wise figures above.
        static = {}
        for cfg, dyn in ((2, (per_call["headwise_fwd"]["avg_us"], per_call["headwise_bwd"]["avg_us"])),
                         (4, (large["headwise-mlp-2b"]["fwd_us"], large["headwise-mlp-2b"]["bwd_us"]))):
            hw = inputs.WORKLOADS[cfg]
            wl = inputs.Workload(hw.name.replace("headwise", "static"), "static", hw.B, hw.T, hw.D, hw.W,
                                 dtype=hw.dtype, residual=hw.residual, cfg=hw.cfg)
            tf, tb, b = fwd_bwd_times(wl, max(5, K // 2))
            static[wl.name] = {"fwd_us": round(tf * 1e6, 1), "bwd_us": round(tb * 1e6, 1),
                               "GBps": round(b / (tf + tb) / 1e9, 1),
                               "frac_hbm_peak": round(b / (tf + tb) / 1e9 / PEAK_HBM_GBPS, 4),
                               "dynamic_headwise_fwd_us": dyn[0], "dynamic_headwise_bwd_us": dyn[1],
                               "dynamic_over_static": round((dyn[0] + dyn[1]) / ((tf + tb) * 1e6), 3)}
        out["static_vs_dynamic"] = static

        # decoding: one new token for each of 64 sequences per step, at the QKV
        # ~150M width (inputs are rows of the step's seeded tensors); the state
        # is updated in place step after step.  us_per_step is a HIP graph of
        # the steps replayed (GPU time); us_per_step_eager launches each step
        # from Python (host-bound at this size)
        S_DEC, STEPS_DEC = 64, 200
        hwc, lrc = cases[0], cases[1]
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
        # workload on the fly; the layer alone is timed in the same loop.  A
        # separate rotation pass would move rot*N elements in and out once
        # more in each direction (unfused_extra_bytes per direction).
        hd, rot = 64, 2 * 768
        table = torch.empty(hwc.wl.T, hd // 2, 2, dtype=torch.float32, device="cuda")
        binding.dsc_rope_table(table, base=10000.0)
        kw = dict(rot=rot, head_dim=hd, table=table, residual=hwc.wl.residual)
        calls = [lambda: binding.dsc_headwise_rope_fwd(hwc.x, hwc.w, hwc.y, **kw),
                 lambda: binding.dsc_headwise_rope_bwd(hwc.x, hwc.w, hwc.dy, hwc.dx, hwc.dw, **kw),
                 hwc.fwd, hwc.bwd]
        for _ in range(3):
            for f in calls:
                f()
        torch.cuda.synchronize()
        reps = max(5, K // 2)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(reps)]
        for e in evs:
            e[0].record()
            for i, f in enumerate(calls):
                f()
                e[i + 1].record()
        torch.cuda.synchronize()
        tr = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / reps * 1e-3 for i in range(len(calls))]
        b = hwc.bytes("fwd") + hwc.bytes("bwd") + 2 * table.numel() * 4
        out["rope_fused"] = {
            "workload": f"{hwc.wl.name} + rotary embedding of channels [0, {rot}), heads of {hd}",
            "fwd_us": round(tr[0] * 1e6, 1), "bwd_us": round(tr[1] * 1e6, 1),
            "GBps": round(b / (tr[0] + tr[1]) / 1e9, 1),
            "frac_hbm_peak": round(b / (tr[0] + tr[1]) / 1e9 / PEAK_HBM_GBPS, 4),
            "layer_alone_fwd_us": round(tr[2] * 1e6, 1), "layer_alone_bwd_us": round(tr[3] * 1e6, 1),
            "unfused_extra_bytes": 2 * rot * hwc.wl.N * hwc.x.element_size()}
        del table

        # The reproducible low-rank backward (dz and dU summed in a fixed order
        # through per-block workspace regions) against the fast one, at the
        # QKV ~150M low-rank size, alternating in the same loop.
    if not args.no_large and not args.no_deterministic:
        lw = lrc.wl
        nws = binding.dsc_lowrank_bwd_deterministic_workspace_size(lrc.x.dtype, lw.B, lw.T, lw.D, lw.W, lw.R)
        det_ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        calls = [lambda: binding.dsc_lowrank_bwd_deterministic(lrc.x, lrc.z, lrc.U, lrc.dy, lrc.dx, lrc.dz, lrc.dU,
                                                               det_ws if nws else None, W=lw.W,
                                                               cu_seqlens=lrc.cu, residual=lw.residual),
                 lrc.bwd]
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
        td = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / reps * 1e-3 for i in range(len(calls))]
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
        td = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / reps * 1e-3 for i in range(len(calls))]
        out["static_bwd_deterministic"] = {
            "workload": swl.name, "us": round(td[0] * 1e6, 1), "fast_us": round(td[1] * 1e6, 1),
            "workspace_bytes": nws}
        del det_ws, sc

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline([cases[0].wl, cases[1].wl], args.cpu_seconds)
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
