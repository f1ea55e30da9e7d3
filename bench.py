"""Benchmark of the MI355X NVFP4 dense SwiGLU FFN (one JSON line on stdout).

A step is one dense_ffn_forward (W4A16: gate+up+silu, down) over one batch
of synthetic rows, inputs resident in HBM.  The headline workload is the
single-row decode FFN (m=1, hidden=4096, inter=12288); the m=64 and
m=2048 workloads the metric also names, the W4A4 and W8A8 fixed-format arms
and the packed-Q2 weights are measured in the same run and reported under
"workloads".

Cold weights: every weight set fits in the 256 MB Infinity Cache, so each
step reads the next of R replicas with R x size >= 1 GiB; the reported
weight GB/s is HBM traffic, not cache hits.

Timing: hipEvents (torch.cuda.Event) recorded on the stream the library
launches on, around exactly K back-to-back steps after W warm-up steps,
bracketed by device synchronizations.

roofline: the dominant kernel is the fused gate+up+silu single-row kernel
k_gemv<1, 2, 1, false> (two thirds of the decode FFN's bytes); its average launch duration
comes from K back-to-back launches of nvfp4_gate_up_silu_w4a16 (one kernel
per call at this shape) between events on the same stream.  Algorithmic
bytes per launch = both weight matrices (codes + E4M3 scales) + x + act.

cpu_baseline: the CPU oracle (fp64, plain loops) on the same decode
workload, repeated for about 10 s on 16 host threads.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
REPLICA_BYTES = 1 << 30
PROFILE_DIR = os.path.join(ROOT, "profiles")
DOMINANT_KERNEL_SRC = os.path.join(ROOT, "nvfp4_weight_dense_amd", "csrc", "k_gemv.hip")
DOMINANT_KERNEL = "k_gemv<1, 2, 1, false>"
TRAFFIC_FILE = os.path.join(PROFILE_DIR, "k_gemv_gate_up_silu_decode_traffic.txt")
COPY_BYTES = 1 << 28


def weight_bytes(w) -> int:
    return int(w.codes.numel() * w.codes.element_size() + w.scales.numel() * w.scales.element_size())


def _replicas(ws, count, device):
    import nvfp4_weight_dense_amd as nv
    out = []
    nvfp4 = hasattr(ws[0], "ts")
    q2 = hasattr(ws[0], "group")
    for _ in range(count):
        if nvfp4:
            out.append([nv.NVFP4Weight(w.codes.to(device, copy=True),
                                       w.scales.to(device, copy=True), w.ts) for w in ws])
        elif q2:
            out.append([nv.Q2Weight(w.codes.to(device, copy=True),
                                    w.scales.to(device, copy=True), w.group) for w in ws])
        else:
            out.append([nv.FP8Weight(w.codes.to(device, copy=True),
                                     w.scales.to(device, copy=True)) for w in ws])
    return out


def _time_loop(fn, reps, steps, warmup, stream):
    import torch
    for i in range(warmup):
        fn(reps[i % len(reps)])
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(reps[i % len(reps)])
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def measure_ffn(name, steps, warmup, w4a4=False, m=None, fused=False, lora_rank=0, w8a8=False,
                q2=False):
    import torch

    import nvfp4_weight_dense_amd as nv
    import synthetic_inputs as si

    dev = torch.device("cuda:0")
    gen = si.fp8_workload if w8a8 else (si.q2_workload if q2 else si.workload)
    x, wg, wu, wd = gen(name, m=m)
    m, hidden = x.shape
    inter = wg.n
    wbytes = weight_bytes(wg) + weight_bytes(wu) + weight_bytes(wd)
    nrep = max(1, math.ceil(REPLICA_BYTES / wbytes))
    xd = x.to(dev)
    out = torch.empty((m, hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    if lora_rank:
        # rank-r pairs on gate, up and down (small: shared by every replica)
        def pair(n, k, which, scale):
            a, b = si.lora_pair(n, k, lora_rank, which=which)
            return nv.LoraPair(a.to(dev), b.to(dev), scale)
        lp = (pair(inter, hidden, 0, 2.0), pair(inter, hidden, 1, -1.5), pair(hidden, inter, 2, 0.5))
        reps = _replicas((wg, wu, wd), nrep, dev)
        fn = lambda xx, g, u, d, out, stream: nv.dense_ffn_forward_lora(xx, g, u, d, *lp, out=out,
                                                                         stream=stream)
    elif fused:
        # one [2*inter, hidden] buffer holding gate then up (same bytes)
        assert wg.ts == wu.ts and not w4a4
        wgu = si.NvWeight(torch.cat([wg.codes, wu.codes]), torch.cat([wg.scales, wu.scales]), wg.ts)
        reps = _replicas((wgu, wd), nrep, dev)
        fn = nv.dense_ffn_forward_fused
    elif w8a8 or q2:
        reps = _replicas((wg, wu, wd), nrep, dev)
        fn = nv.dense_ffn_forward_w8a8 if w8a8 else nv.dense_ffn_forward_q2
    else:
        reps = _replicas((wg, wu, wd), nrep, dev)
        fn = nv.dense_ffn_forward_w4a4 if w4a4 else nv.dense_ffn_forward
    ms = _time_loop(lambda r: fn(xd, *r, out=out, stream=stream), reps, steps, warmup, stream)
    flops = 6.0 * m * hidden * inter
    res = {
        "workload": f"{name} m={m} hidden={hidden} inter={inter}" + (" w4a4" if w4a4 else "")
                    + (" (block-scaled FP8 weights, per-row FP8 activations)" if w8a8 else "")
                    + (" (packed-Q2 weights, group 128, bf16 activations)" if q2 else "")
                    + (" fused gate+up weight" if fused else "")
                    + (f" + LoRA rank {lora_rank} on gate, up, down" if lora_rank else ""),
        "m": m, "hidden": hidden, "inter": inter,
        "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "weight_gbs": wbytes / (ms * 1e-3) / 1e9,
        "weight_bytes": wbytes,
        "replicas": nrep,
    }
    res["hbm_frac"] = res["weight_gbs"] / HBM_PEAK_GBS
    res["mfma_frac"] = res["tflops"] / (FP8_PEAK_TFLOPS if w8a8 else BF16_PEAK_TFLOPS)
    ctx = dict(x=xd, weights=reps, out=out, stream=stream, wbytes=wbytes)
    return res, ctx


def measure_dominant_kernel(ctx, steps, warmup):
    """Average duration of the fused gate+up+silu launch at the decode shape."""
    import torch

    import nvfp4_weight_dense_amd as nv

    xd, reps, stream = ctx["x"], ctx["weights"], ctx["stream"]
    m = xd.shape[0]
    inter = reps[0][0].codes.shape[0]
    act = torch.empty((m, inter), dtype=torch.bfloat16, device=xd.device)
    ms = _time_loop(lambda r: nv.nvfp4_gate_up_silu_w4a16(xd, r[0], r[1], act=act, stream=stream),
                    reps, steps, warmup, stream)
    algo = (weight_bytes(reps[0][0]) + weight_bytes(reps[0][1])
            + xd.numel() * 2 + act.numel() * 2)
    achieved = algo / (ms * 1e-3) / 1e9
    return {
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": achieved / HBM_PEAK_GBS,
        "traffic": _traffic_per_launch(),
        "kernel": DOMINANT_KERNEL + " (nvfp4_gate_up_silu_w4a16, m=1, k=4096, n=12288)",
        "avg_launch_us": ms * 1e3,
        "algorithmic_bytes": algo,
    }


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in (DOMINANT_KERNEL_SRC,
              os.path.join(ROOT, "nvfp4_weight_dense_amd", "csrc", "nvfp4_common.h")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic_per_launch():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on the kernel source as it is now."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("source_hash") != _kernel_source_hash():
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def traffic_run(steps, what="gemv"):
    """Launch pattern for the rocprofv3 FETCH_SIZE / WRITE_SIZE passes: `steps`
    launches of the dominant kernel over rotating cold replicas (what="gemv"),
    or `steps` whole decode FFNs in the W4A4 or W8A8 ("w4a4", "w8a8": m=1,
    hidden 4096, inter 14336) or packed-Q2 ("q2", m=1, hidden 4096, inter
    12288) formats, then
    `steps` plain device copies of COPY_BYTES, whose counter readings
    calibrate the counters against a transfer of known size."""
    import torch

    import nvfp4_weight_dense_amd as nv

    if what == "gemv":
        _, ctx = measure_ffn("decode", 1, 1)
    elif what == "w4a4":
        _, ctx = measure_ffn("w4a4", 1, 1, m=1, w4a4=True)
    else:
        _, ctx = measure_ffn("w8a8" if what == "w8a8" else "decode", 1, 1, m=1,
                             w8a8=what == "w8a8", q2=what == "q2")
    xd, reps, stream = ctx["x"], ctx["weights"], ctx["stream"]
    act = torch.empty((xd.shape[0], reps[0][0].codes.shape[0]), dtype=torch.bfloat16,
                      device=xd.device)
    out = ctx["out"]
    for i in range(steps):
        r = reps[i % len(reps)]
        if what == "gemv":
            nv.nvfp4_gate_up_silu_w4a16(xd, r[0], r[1], act=act, stream=stream)
        elif what == "w8a8":
            nv.dense_ffn_forward_w8a8(xd, *r, out=out, stream=stream)
        elif what == "w4a4":
            nv.dense_ffn_forward_w4a4(xd, *r, out=out, stream=stream)
        else:
            nv.dense_ffn_forward_q2(xd, *r, out=out, stream=stream)
    torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=xd.device)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_run": DOMINANT_KERNEL if what == "gemv" else what, "launches": steps,
                      "copy_bytes": COPY_BYTES, "source_hash": _kernel_source_hash()}),
          flush=True)


def cpu_baseline(seconds=10.0, threads=16):
    import numpy as np

    import oracle
    import synthetic_inputs as si

    x, wg, wu, wd = si.workload("decode")
    ow = [oracle.Weight(w.codes.numpy(), w.scales.numpy(), w.ts) for w in (wg, wu, wd)]
    xb = x.view(__import__("torch").int16).numpy().view(np.uint16)
    threads = max(1, min(threads, os.cpu_count() or 1))
    wbytes = sum(weight_bytes(w) for w in (wg, wu, wd))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.dense_ffn(xb, *ow, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or el > 30:
            break
    return {
        "value": wbytes * reps / el / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps} full decode FFNs (m=1, hidden=4096, inter=12288) in {el:.1f} s",
        "ms_per_step": el / reps * 1e3,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed calls before the timed ones (about 10 ms of decode work: "
                         "kernels in the first ~40 ms of a process run slower)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-headline", action="store_true",
                    help="time only the decode workload (for profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--traffic-run", nargs="?", const="gemv", default=None,
                    choices=("gemv", "w4a4", "w8a8", "q2"),
                    help="only launch the dominant kernel (or a W8A8 / packed-Q2 decode FFN) "
                         "and a calibration copy (for rocprofv3 --pmc passes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the FFN runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch

    import nvfp4_weight_dense_amd as nv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    nv.load_library()  # raises if the HIP library is not built
    if args.traffic_run:
        traffic_run(args.steps, args.traffic_run)
        return

    head, ctx = measure_ffn("decode", args.steps, args.warmup)
    roof = measure_dominant_kernel(ctx, args.steps, args.warmup)
    del ctx
    workloads = []
    if not args.only_headline:
        for name, steps, w4a4, m, fused, rank, q2 in (
                ("decode", args.steps, False, None, False, 0, True),
                ("smallm", max(20, args.steps // 2), False, None, False, 0, True),
                ("prefill", max(5, args.steps // 20), False, None, False, 0, True)):
            r, c = measure_ffn(name, steps, max(3, args.warmup // 2), q2=q2)
            del c
            torch.cuda.empty_cache()
            workloads.append(r)
        for name, steps, w4a4, m, fused, rank in (
                ("decode", args.steps, False, None, True, 0),
                ("decode", args.steps, False, None, False, 16),
                ("smallm", max(20, args.steps // 2), False, None, False, 0),
                ("prefill", max(5, args.steps // 20), False, None, False, 0),
                ("decode_tp8", args.steps, False, None, False, 0),
                ("prefill_tp8", max(5, args.steps // 20), False, None, False, 0),
                ("w4a4", max(20, args.steps // 2), True, 1, False, 0),
                ("w4a4", max(20, args.steps // 2), True, 8, False, 0),
                ("w4a4", max(20, args.steps // 2), True, 64, False, 0),
                ("w4a4", max(5, args.steps // 20), True, 512, False, 0),
                ("w8a8", max(20, args.steps // 2), False, 1, False, 0),
                ("w8a8", max(20, args.steps // 2), False, 8, False, 0),
                ("w8a8", max(20, args.steps // 2), False, 64, False, 0),
                ("w8a8", max(5, args.steps // 20), False, 512, False, 0)):
            r, c = measure_ffn(name, steps, max(3, args.warmup // 2), w4a4=w4a4, m=m, fused=fused,
                               lora_rank=rank, w8a8=name == "w8a8")
            del c
            torch.cuda.empty_cache()
            workloads.append(r)
    nv.nvfp4_release()
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)

    line = {
        "metric": "dense FFN TFLOP/s + weight HBM GB/s (% roofline) at m=1/64/2048, 1 MI355X",
        "value": head["weight_gbs"],
        "unit": "GB/s (NVFP4 weight bytes / s)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "m": head["m"], "hidden": head["hidden"], "inter": head["inter"],
            "weights": "NVFP4 (E2M1 + E4M3/16 + fp32 tensor scale)",
            "accumulate": "fp32",
            "cold_weight_replicas": head["replicas"],
        },
        "tflops": head["tflops"],
        "hbm_frac": head["hbm_frac"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
