#!/usr/bin/env python3
"""Forward + full VJP of ragged extreme-GQA attention on one MI355X.

One step = one attn_varlen_full_vjp call (plan, forward with the dO.O row dot,
dK/dV with stored dS, dQ with the partial sums) over the resident synthetic
batch, with the workspace sized so every sequence's dS is stored.  The default
workload is the Hq=64 Q-short/K-long configuration: 24 sequences, Lq ~ U[16,128],
Lk ~ U[512,2048], one K/V head, D = 160, BF16 views of width 192 with token step 2.

Prints one JSON line.  `value` is credited TFLOP/s = 14 * sum_b Lq_b Lk_b * Hq * D
per call / time per call, over K plain calls.  The kernels skip the 64-key steps
in which every probability of a 256-row tile is exactly zero (far from the ALiBi
centre under the soft cap); `evaluated_pair_fraction` is the share of the
credited (row, key) pairs that the forward and dQ row tiles evaluate, read back
from the library after the timed loops.  `roofline` covers the kernel with the
longest average duration, timed by a loop of K calls (run just before the
headline loop) with HIP events recorded on the library's stream before each
phase; its `achieved` is credited FLOPs / duration, and `achieved_executed`
scales it by the evaluated fraction (the matrix work the kernel really does).
`kernels` puts each kernel against its own roof: the forward and dK/dV against
the MFMA peak, dQ (which reads the stored dS images) against HBM, with the
fabric bytes of the committed traffic summary when it matches the sources.
`cpu_baseline` times the float64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+full-VJP TFLOP/s (% MFMA peak) and ms/call, ragged GQA Hq=64 D=160"
MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense FP16/BF16 matrix peak
HBM_PEAK_TBPS = 8.0           # MI355X HBM3E
# credited flops per score element and head-dim unit, by phase (14 in total)
PHASE_FLOPS = {"fwd": 4, "dkdv": 8, "dq": 2, "plan": 0}


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "ragged_gqa_attention_amd", "csrc", "*"))):
        if path.endswith((".hip", ".hpp", ".cpp")):
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the summary is missing or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    d = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m or not d or d.group(1) != kernel_source_digest():
        return None
    return float(m.group(1))


def measured_kernel_bytes(workload: str):
    """Fabric bytes (read, written) per launch of each kernel from the committed
    traffic summary, or None when it is missing or the kernels changed."""
    path = os.path.join(ROOT, "profiles", f"dkdv_kernel_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    d = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not d or d.group(1) != kernel_source_digest():
        return None
    rows = re.findall(r"^\| `(\w+)<[^`]*>` \| [0-9.]+ \| [0-9.]+ \| ([0-9.]+) \| ([0-9.]+) \|",
                      text, re.M)
    return {k: (float(r) * 1e6, float(w) * 1e6) for k, r, w in rows} or None


def measured_busy(kernel: str, workload: str):
    """Per-unit busy fractions of a kernel (MFMA, VALU, their co-issue, LDS)
    from the committed SQ counter summary, or None when it is missing or the
    kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"sq_counters_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    d = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m = re.search(rf"busy {kernel}: mfma=([0-9.]+) valu=([0-9.]+) coissue=([0-9.]+) lds=([0-9.]+)"
                  rf" clock_mhz=([0-9.]+)", text)
    if not m or not d or d.group(1) != kernel_source_digest():
        return None
    keys = ("mfma", "valu", "coissue", "lds")
    out = {k: float(v) for k, v in zip(keys, m.groups()[:4])}
    out["clock_mhz"] = float(m.group(5))
    return out


def cpu_baseline(wl, seconds: float):
    """The float64 oracle, unchanged, on the first sequences of the workload
    until about `seconds` of CPU time."""
    import oracle
    from workloads import oracle_inputs
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "version": i.get("version"),
                 "threads": i.get("num_threads"), "arch": i.get("architecture")}
                for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover - threadpoolctl is optional
        pass
    # NumPy's elementwise steps run on one thread; its matrix products use the
    # BLAS pool, so the pool's size is the most threads the oracle can use
    threads = max([b["threads"] or 1 for b in blas] + [1])
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    inp = oracle_inputs(wl)
    cu_q, cu_k = inp["cu_q"], inp["cu_k"]
    spent, elems, n = 0.0, 0, 0
    for b in range(wl.batch):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        t0 = time.perf_counter()
        oracle.sequence_vjp(inp["q"][q0:q1], inp["k"][k0:k1], inp["v"][k0:k1],
                            inp["dout"][q0:q1], inp["alibi_slopes"][b], inp["softcap"],
                            inp["scale_multiplier"])
        spent += time.perf_counter() - t0
        elems += (q1 - q0) * (k1 - k0) * wl.hq
        n += 1
        if spent >= seconds:
            break
    flops = 14.0 * elems * wl.head_dim
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model, "os_cpu_count": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "blas": blas,
            "sample": f"first {n} of {wl.batch} sequences of {wl.name} "
                      f"(sum Lq*Lk*Hq = {elems}), float64 NumPy forward + VJP, "
                      f"{spent:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # the first ~50 calls run measurably slower (the GPU is still ramping up),
    # so the default warm-up is long enough to time the steady state
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=1,
                    help="workload index (1 = the Hq=64 metric configuration)")
    ap.add_argument("--trial", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--causal", action="store_true", help="bottom-right causal mask")
    ap.add_argument("--window", type=int, nargs=2, default=(-1, -1), metavar=("LEFT", "RIGHT"),
                    help="sliding window bounds (-1 = none)")
    ap.add_argument("--dropout-p", type=float, default=0.0,
                    help="counter-based dropout rate (0 = none, the configurations' setting)")
    ap.add_argument("--dropout-seed", type=int, default=1234)
    ap.add_argument("--recompute-ds", action="store_true",
                    help="dQ rebuilds dS instead of reading the dK/dV kernel's stored images")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the "
              "path is one GPU's share of the batch and no multi-GPU sharding is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import ragged_gqa_attention_amd as rga
    from ragged_gqa_attention_amd import _lib
    from workloads import make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = make_workload(args.config, args.trial)
    g = wl.to(dev)
    call = rga.FullVJP(g.q, g.k, g.v, g.cu_q, g.cu_k, g.slopes, g.dout, softcap=g.softcap,
                       scale_multiplier=g.scale_multiplier, store_ds=not args.recompute_ds,
                       causal=args.causal, window_left=args.window[0],
                       window_right=args.window[1],
                       dropout_p=args.dropout_p, dropout_seed=args.dropout_seed)
    nph = len(_lib.PHASES)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    call.check_plan()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(K)]
    for row in evs:          # creates the underlying HIP events
        for e in row:
            e.record()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # timed region 1: K calls with an event recorded on the library's stream
    # before each phase: per-phase and per-call durations (the records add a
    # few microseconds per call, so the headline comes from region 2)
    torch.cuda.synchronize()
    for i in range(K):
        call(events=evs[i])
    torch.cuda.synchronize()
    per_call = np.array([evs[i][0].elapsed_time(evs[i][nph]) for i in range(K)])
    # timed region 2: K plain calls (the headline figure)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(K):
        call()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / K
    phase_ms = {name: float(np.mean([evs[i][p].elapsed_time(evs[i][p + 1]) for i in range(K)]))
                for p, name in enumerate(_lib.PHASES)}

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    elems = wl.score_elements()
    if args.causal or args.window[0] >= 0 or args.window[1] >= 0:
        # a mask removes pairs from the work: credit only the kept ones
        wr_ = 0 if args.causal else args.window[1]
        wl_ = args.window[0]
        kept = 0
        for lq, lk in zip(wl.lq, wl.lk):
            c = np.arange(int(lq)) + int(lk) - int(lq)
            lo = np.maximum(0, c - wl_) if wl_ >= 0 else np.zeros_like(c)
            hi = np.minimum(int(lk) - 1, c + wr_) if wr_ >= 0 else np.full_like(c, int(lk) - 1)
            kept += int(np.maximum(hi - lo + 1, 0).sum())
        elems = kept * wl.hq
    flops = 14.0 * elems * wl.head_dim
    # share of the credited (row, key) pairs inside the recorded key-step ranges
    ks = call.key_steps().astype(np.int64)
    evaluated = 0
    tile = 0
    group = wl.hq // wl.hkv   # rows of one K/V head's query heads fold together
    for lq, lk in zip(wl.lq, wl.lk):
        rows = int(lq) * group
        for _ in range(wl.hkv):
            for t0 in range(0, rows, 256):
                lo, hi = ks[tile]
                tile += 1
                evaluated += min(256, rows - t0) * max(0, min(int(hi) * 64, int(lk)) - int(lo) * 64)
    frac = evaluated / elems if elems else 1.0
    value = flops / (ms_per_step * 1e-3) / 1e12
    dom = max(("fwd", "dkdv", "dq"), key=lambda p: phase_ms[p])
    achieved = PHASE_FLOPS[dom] * elems * wl.head_dim / (phase_ms[dom] * 1e-3) / 1e12
    kernel_names = {"fwd": "fwd_kernel", "dkdv": "dkdv_kernel", "dq": "dq_kernel"}
    traffic = measured_traffic(kernel_names[dom], wl.name)
    busy = measured_busy(kernel_names[dom], wl.name)
    # what holds the kernel below the MFMA roof, from its SQ counters: the
    # unit with the larger busy share (the two overlap only by `coissue`)
    limiter = None
    if busy is not None:
        limiter = "valu" if busy["valu"] > busy["mfma"] else "mfma"
    # every kernel against its own roof: the forward and dK/dV do far more
    # matrix work per byte than the MI355X ridge (2500 TFLOP/s / 8 TB/s), dQ
    # with stored dS does 2 D flops per 2-byte dS element read, below it
    kbytes = measured_kernel_bytes(wl.name)
    kernels = {}
    for ph in ("fwd", "dkdv", "dq"):
        name = kernel_names[ph]
        t = phase_ms[ph] * 1e-3
        tf = PHASE_FLOPS[ph] * elems * wl.head_dim / t / 1e12
        e = {"ms": round(phase_ms[ph], 4), "credited_tflops": round(tf, 3),
             "mfma_frac": round(tf / MFMA_PEAK_TFLOPS, 5)}
        hbm = ph == "dq" and not args.recompute_ds
        if kbytes and name in kbytes:
            rd, wr = kbytes[name]
            e["fabric_tbps"] = round((rd + wr) / t / 1e12, 3)
            e["fabric_bytes"] = int(rd + wr)
        elif hbm:
            # algorithmic bytes: the dS images read (2 B per evaluated element)
            # and dQ written
            byts = 2.0 * elems * frac + 2.0 * wl.total_q * wl.hq * wl.head_dim
            e["fabric_tbps"] = round(byts / t / 1e12, 3)
            e["fabric_bytes"] = None
        e["bound"] = "hbm" if hbm else "mfma"
        if hbm:
            e["frac"] = round(e["fabric_tbps"] / HBM_PEAK_TBPS, 5)
        else:
            e["frac"] = e["mfma_frac"]
        kernels[name] = e
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "seed": [args.config, args.trial], "batch": wl.batch,
            "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.head_dim, "total_q": wl.total_q,
            "total_k": wl.total_k, "sum_lq_lk": int((wl.lq * wl.lk).sum()),
            "view": f"feature width {wl.width}, token step {wl.step}",
            "softcap": wl.softcap, "scale_multiplier": wl.scale_multiplier,
            "dropout_p": args.dropout_p, "causal": args.causal, "window": list(args.window),
            "stored_ds": not args.recompute_ds,
        },
        "pct_mfma_peak": round(100.0 * value / MFMA_PEAK_TFLOPS, 3),
        "ms_per_call_median": round(float(np.median(per_call)), 4),
        "host_wall_ms_per_step": round(1e3 * wall / K, 4),
        "phase_ms": {k: round(v, 4) for k, v in phase_ms.items()},
        "evaluated_pair_fraction": round(frac, 4),
        "roofline": {
            "kernel": kernel_names[dom],
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_PEAK_TFLOPS, 5),
            "achieved_executed": round(achieved * frac, 3),
            "traffic": traffic,
            "limiter": limiter,
            "busy": busy,
        },
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
