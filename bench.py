#!/usr/bin/env python3
"""Benchmark of K-interval attention forward + backward on one MI355X.

One step = kia_forward + kia_backward (full calibration gradients) for each of
the six operator variants of the GPT-2-124M attention workload
(B=8, H=12, T=1024, D=64, causal, fp32 N(0,1) inputs, seed 1):
{MinMax, FWM tau=8} x {LERP, Nearest + Weight-STE, Nearest + Prob-STE}, K=4.
Together they run every stage of the hot path (scores, extrema, grid table,
reconstruction, normalization, P V, D_i, surrogate gamma, calibration sums,
dV / dK / dQ, calibration gradient at the arg-max / arg-min keys).

value = algorithmic TFLOP/s over the whole step: 12 D flops per causal
(query, key) pair per variant (forward QK^T + PV = 4D, backward dP, dV, dK,
dQ = 8D), divided by the wall time of the timed steps (inputs resident in HBM).
Per-kernel times come from HIP events recorded on the stream the kernels are
launched on; the roofline object is for the kernel that takes the most time.

Prints ONE JSON line on stdout; details on stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "K-interval attn fwd+bwd TFLOP/s & % MFMA peak, B=8 H=12 T=1024 d=64 causal"
FP32_MFMA_PEAK = 157.3   # TFLOP/s, MI355X dense fp32 matrix
BF16_MFMA_PEAK = 2500.0
# algorithmic flops per causal pair, in units of D, per kernel
ALG_PER_PAIR = {"fwd": 4, "dq": 4, "dkdv": 4, "bwd": 8, "fwd1": 2, "fwd2": 2}
KERNEL_SOURCES = ["kia_device.hpp", "kia_launch.hpp", "kia_fwd.hip", "kia_bwd.hip", "kia_api.hip", "kia_flash.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantized_softmax_attention_kia_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str = "gpt2"):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/hbm_traffic_<workload>_fwd_bwd.md),
    or None when there are none or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}_fwd_bwd.md")
    if not os.path.exists(path):
        return None
    digest = sources_digest()
    for line in open(path):
        parts = line.split()
        # machine-readable lines:  traffic <kernel> <bytes_per_launch> <sources_digest>
        if len(parts) == 4 and parts[0] == "traffic" and parts[1] == kernel and parts[3] == digest:
            return float(parts[2])
    return None


def read_issue(kernel: str, workload: str = "gpt2"):
    """SQ counters of the kernel (profiles/sq_counters_<workload>_fwd_bwd.md): the VALU's and the
    matrix pipe's busy shares of SIMD time and the waves' share of time waiting, or None when there
    are none or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"sq_counters_{workload}_fwd_bwd.md")
    if not os.path.exists(path):
        return None
    digest = sources_digest()
    for line in open(path):
        parts = line.split()
        # machine-readable lines:  issue <kernel> <valu_busy> <mfma_busy> <wait_any> <sources_digest>
        if len(parts) == 6 and parts[0] == "issue" and parts[1] == kernel and parts[5] == digest:
            valu, mfma, wait = (float(x) for x in parts[2:5])
            return {"limiter": "valu" if valu > mfma else "mfma", "valu_busy": valu, "mfma_busy": mfma,
                    "wait_any": wait}
    return None


def cpu_baseline(variants, q, k, v, do, budget_s: float, grad: str = "full", threads: int = 0):
    """The oracle, as it stands, on a bounded sample: heads in order, every variant, until the budget
    (on `threads` host threads; 0: all of them)."""
    import dataclasses
    from oracle import oracle as ORC
    threads = threads or ORC.default_threads()
    B, H, T, D = q.shape
    pairs = T * (T + 1) // 2
    done_heads, flops = 0, 0.0
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(H):
            for var in variants:
                cfg = dataclasses.replace(ORC.OracleConfig.of(var), grad=grad)
                ORC.head(cfg, q[b, h], k[b, h], v[b, h], do[b, h], nthreads=threads)
                flops += 12.0 * D * pairs
            done_heads += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        else:
            continue
        break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done_heads} of {B * H} heads of the same workload, all {len(variants)} variants, "
                      f"forward+backward in double, {dt:.1f} s wall"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--grad", default="full", choices=["full", "detached", "max_only", "min_only", "p1"],
                    help="gradient mode of every variant (the headline is full)")
    ap.add_argument("--tail", default="zero", choices=["zero", "floor", "resolved"],
                    help="tail policy of the FWM variants (the headline is zero, the FWM of the pages)")
    ap.add_argument("--binmean", action="store_true",
                    help="time bin mean and the Nearest-forward / bin-mean-backward hybrid (MinMax and FWM, "
                         "K = 4) on the same workload instead of the K-interval variants")
    ap.add_argument("--baselines", action="store_true",
                    help="time the one-pass (online-rescale) exact softmax beside the K-interval variants and "
                         "the exponential baselines (softmax, BF16-exp, FP8-rounded exp) on the two-pass "
                         "pipeline, on the same workload")
    ap.add_argument("--split-forward", action="store_true",
                    help="run the forward as its two launches (kia_forward_scores: scores and exact extrema; "
                         "kia_forward_weights: calibration, reconstruction, normalization, P V) and time each")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (a known-size reference for HBM "
                         "byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the implementation runs on one GPU; --gpus {args.gpus} is not supported "
              "(the operator would shard over batch x heads with no exchange between GPUs)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from quantized_softmax_attention_kia_amd import binding as kb
    from quantized_softmax_attention_kia_amd.inputs import WORKLOADS

    import dataclasses
    wl = WORKLOADS[args.workload]
    variants = [dataclasses.replace(v, tail=args.tail) if v.calib == "fwm" else v for v in wl.variants]
    if args.baselines:
        from quantized_softmax_attention_kia_amd.inputs import Variant
        variants = variants + [Variant("fwm", r, "prob", "full", 4) for r in ("softmax", "exp_bf16", "exp_fp8")]
        variants.append("flash-softmax")
    if args.binmean:
        from quantized_softmax_attention_kia_amd.inputs import Variant
        variants = [Variant(c, r, "prob", "full", 4) for c in ("minmax", "fwm") for r in ("binmean", "nearest_binmean")]
    log(f"workload {wl.name}: B={wl.B} H={wl.H} T={wl.T} D={wl.D} {wl.dtype} seed={wl.seed}; "
        f"{len(variants)} variants")
    q, k, v, do = wl.inputs()
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    qt, kt, vt, dot = (torch.from_numpy(x).to(dev).to(tdt) for x in (q, k, v, do))
    stream = torch.cuda.current_stream()

    runs = []
    for var in variants:
        if var == "flash-softmax":
            cfg = kb.Config("fwm", "softmax", "prob", "full", 4)
            p = kb.make_params(cfg, qt.shape, tdt)
            runs.append(dict(
                name="flash-softmax", kind="flash", p=p,
                o=torch.empty(qt.shape, device=dev, dtype=torch.float32),
                rowstats=torch.empty(3 * wl.B * wl.H * wl.T, device=dev, dtype=torch.float32),
                dq=torch.empty(qt.shape, device=dev, dtype=torch.float32),
                dk=torch.empty(qt.shape, device=dev, dtype=torch.float32),
                dv=torch.empty(qt.shape, device=dev, dtype=torch.float32)))
            continue
        cfg = kb.Config.of(var)
        if args.grad != cfg.grad:
            cfg = dataclasses.replace(cfg, grad=args.grad)
        p = kb.make_params(cfg, qt.shape, tdt)
        rr, ws = kb.kia_workspace_size(p)
        runs.append(dict(
            name=var.name if args.grad == "full" else f"{var.name}:{args.grad}", kind="kia", p=p,
            o=torch.empty(qt.shape, device=dev, dtype=torch.float32),
            rowrec=torch.empty(max(rr, 1), device=dev, dtype=torch.uint8),
            dq=torch.empty(qt.shape, device=dev, dtype=torch.float32),
            dk=torch.empty(qt.shape, device=dev, dtype=torch.float32),
            dv=torch.empty(qt.shape, device=dev, dtype=torch.float32),
            ws=torch.empty(max(ws, 1), device=dev, dtype=torch.uint8)))

    def one_step(events=None):
        for i, r in enumerate(runs):
            if r["kind"] == "flash":
                if events is not None:
                    events[i][0].record(stream)
                kb.kia_flash_forward(r["p"], qt, kt, vt, r["o"], r["rowstats"], stream)
                if events is not None:
                    events[i][1].record(stream)
                kb.kia_flash_backward(r["p"], qt, kt, vt, r["o"], dot, r["rowstats"], r["dq"], r["dk"], r["dv"], stream)
                if events is not None:
                    events[i][2].record(stream)
                    events[i][3].record(stream)
                continue
            if events is not None:
                events[i][0].record(stream)
            if args.split_forward:
                kb.kia_forward_scores(r["p"], qt, kt, vt, r["rowrec"], stream)
                if events is not None:
                    events[i][4].record(stream)
                kb.kia_forward_weights(r["p"], qt, kt, vt, r["o"], r["rowrec"], stream)
            else:
                kb.kia_forward(r["p"], qt, kt, vt, r["o"], r["rowrec"], stream)
            if events is not None:
                events[i][1].record(stream)
            kb.kia_backward_dq(r["p"], qt, kt, vt, r["o"], dot, r["rowrec"], r["dq"], r["ws"], stream)
            if events is not None:
                events[i][2].record(stream)
            kb.kia_backward_dkdv(r["p"], qt, kt, vt, dot, r["rowrec"], r["dk"], r["dv"], r["ws"], stream)
            if events is not None:
                events[i][3].record(stream)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calibrate_copy} MiB read, {args.calibrate_copy} MiB written")
        del src, dst

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()

    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev = [[[mk() for _ in range(5)] for _ in runs] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_step(ev[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    pairs = wl.causal_pairs
    alg_flops_variant = 12.0 * wl.D * pairs
    step_flops = alg_flops_variant * len(runs)
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    peak = BF16_MFMA_PEAK if wl.dtype == "bf16" else FP32_MFMA_PEAK

    # per-kernel average launch durations from the events
    per = {}
    for i, r in enumerate(runs):
        split = args.split_forward and r["kind"] == "kia"
        stages = ("fwd", "bwd") if r["kind"] == "flash" else (("fwd1", "fwd2") if split else ("fwd",)) + ("dq", "dkdv")
        durs = {st: [] for st in stages}
        for s in range(args.steps):
            e = ev[s][i]
            if split:
                durs["fwd1"].append(e[0].elapsed_time(e[4]))
                durs["fwd2"].append(e[4].elapsed_time(e[1]))
            else:
                durs["fwd"].append(e[0].elapsed_time(e[1]))
            if r["kind"] == "flash":
                durs["bwd"].append(e[1].elapsed_time(e[2]))
            else:
                durs["dq"].append(e[1].elapsed_time(e[2]))
                durs["dkdv"].append(e[2].elapsed_time(e[3]))
        per[r["name"]] = {kname: float(np.mean(x)) for kname, x in durs.items()}
    for name, d in per.items():
        tot = sum(d.values())
        log(f"  {name:32s} " + "  ".join(f"{st} {x:.3f} ms" for st, x in d.items()) +
            f"  total {tot:.3f} ms  -> {alg_flops_variant / (tot * 1e-3) / 1e12:.1f} TFLOP/s")
    baselines = None
    if args.baselines:
        fl = sum(per["flash-softmax"].values())
        kint = [n for n, r in zip(per, runs) if r["kind"] == "kia" and r["p"].recon in (0, 1)]
        baselines = {"flash_softmax_ms": round(fl, 4),
                     "flash_softmax_tflops": round(alg_flops_variant / (fl * 1e-3) / 1e12, 3),
                     "time_over_flash_softmax": {n: round(sum(per[n].values()) / fl, 3) for n in per
                                                 if n != "flash-softmax"}}
        log(f"one-pass exact softmax {fl:.3f} ms; K-interval variants take "
            + ", ".join(f"{sum(per[n].values()) / fl:.2f}x" for n in kint) + " of it")
    # dominant kernel: the (variant, stage) launch with the largest average duration
    dom_var, dom_stage = max(((n, st) for n in per for st in per[n]), key=lambda x: per[x[0]][x[1]])
    dom_ms = per[dom_var][dom_stage]
    dom_alg = ALG_PER_PAIR[dom_stage] * wl.D * pairs
    achieved = dom_alg / (dom_ms * 1e-3) / 1e12
    kernel_key = f"{dom_stage}:{dom_var}"
    # the committed counters are of each workload's default step
    default_step = (args.grad == "full" and args.tail == "zero" and not args.baselines
                    and not args.binmean and not args.split_forward)
    traffic = read_traffic(kernel_key, args.workload) if default_step else None
    issue = read_issue(kernel_key, args.workload) if default_step else None
    slowest = max(per, key=lambda n: sum(per[n].values()))
    slowest_tflops = alg_flops_variant / (sum(per[slowest].values()) * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms; {value:.1f} TFLOP/s = {100 * value / peak:.1f}% of {peak} TFLOP/s; "
        f"slowest variant {slowest} {slowest_tflops:.1f} TFLOP/s; dominant kernel {kernel_key} {dom_ms:.3f} ms")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a bounded sample ...")
        kv = [x for x in variants if not isinstance(x, str)]
        cpu = cpu_baseline(kv, q, k, v, do, args.cpu_seconds, args.grad)
        # the same oracle on one host thread, over a shorter sample
        one = cpu_baseline(kv, q, k, v, do, max(1.0, args.cpu_seconds / 4), args.grad, threads=1)
        cpu["one_core"] = {"value": one["value"], "unit": one["unit"], "sample": one["sample"]}
        log(f"cpu baseline {cpu}")

    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: B={wl.B} H={wl.H} T={wl.T} D={wl.D} causal {wl.dtype} N(0,1) seed {wl.seed}; "
                        f"one step = fwd+bwd ({args.grad} calibration gradients) of "
                        + ", ".join(r["name"] for r in runs),
            "B": wl.B, "H": wl.H, "T": wl.T, "D": wl.D, "causal": True,
            "alg_flops_per_step": step_flops,
            "frac_of_mfma_peak": round(value / peak, 4),
            # the same step priced by the FlashAttention convention, 14 D flops per causal pair (4 D
            # forward; 10 D backward, the recomputed Q K^T included), for comparison with such figures
            "flash_convention_tflops": round(value * 14.0 / 12.0, 3),
            "slowest_variant": {"name": slowest, "tflops": round(slowest_tflops, 3),
                                "ms": round(sum(per[slowest].values()), 4)},
            "kernel_ms": {n: {k2: round(x, 4) for k2, x in d.items()} for n, d in per.items()},
            "baselines": baselines,
        },
        "roofline": {"bound": "mfma", "kernel": kernel_key, "achieved": round(achieved, 3),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "issue": issue},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
