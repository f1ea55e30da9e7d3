"""Benchmark of the MI355X NVFP4 dense SwiGLU FFN (one JSON line on stdout).

A step is one dense_ffn_forward (W4A16: gate+up+silu, down) over one batch
of synthetic rows, inputs resident in HBM.  The headline workload is the
single-row decode FFN (m=1, hidden=4096, inter=12288); the m=64 and
m=2048 workloads the metric also names, the W4A4 and W8A8 fixed-format arms
and the packed-Q2 weights are measured in the same run and reported under
"workloads".

Cold weights: every weight set fits in the 256 MB Infinity Cache, so each
step reads the next of R replicas with R x size >= 1 GiB; the reported
weight GB/s is HBM traffic, not cache hits.  "warm" entries (one replica,
cache-resident) are measured separately and labelled as such.

Timing: hipEvents (torch.cuda.Event) recorded on the stream the library
launches on, around exactly K back-to-back steps after W warm-up steps,
bracketed by device synchronizations.  Before the W warm-up steps of each
workload the same call runs untimed for RAMP_S seconds of wall time: after
an idle gap (weight replicas being built on the host) the first tens of
milliseconds of GPU work run up to 20% slower, and a warm-up counted in
calls would time that ramp instead of the kernels.

roofline: the dominant kernel is the fused gate+up+silu single-row kernel
k_gemv<1, 2, 1, false> (two thirds of the decode FFN's bytes); its average
launch duration comes from K back-to-back launches of
nvfp4_gate_up_silu_w4a16 (one kernel per call at this shape) between events
on the same stream.  Algorithmic bytes per launch = both weight matrices
(codes + E4M3 scales) + x + act.

mfma_peak: the bf16 matrix throughput a register-only MFMA loop reaches on
this part (nvfp4_probe_mfma_bf16), beside the 2.5 PFLOP/s specification.

cpu_baseline: the CPU oracle (fp64, plain loops) on the same decode
workload, repeated for about 10 s on the host's cores; per_config: the
oracle on a few sampled rows of every workload (its time scaled to the
workload's rows, and the GPU rows' max |err| / rms against it).
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
RAMP_S = 0.15                   # untimed calls before the counted warm-up, per workload
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


def _ramp(fn, reps, seconds):
    """Untimed calls for `seconds` of wall time (GPU clock ramp)."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn(reps[i % len(reps)])
            i += 1
        torch.cuda.synchronize()
    return i


def _time_loop(fn, reps, steps, warmup, stream, ramp_s=RAMP_S):
    import torch
    _ramp(fn, reps, ramp_s)
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


def _label(name, m, hidden, inter, w4a4=False, w8a8=False, q2=False, fused=False, lora_rank=0,
           warm=False):
    return (f"{name} m={m} hidden={hidden} inter={inter}" + (" w4a4" if w4a4 else "")
            + (" (block-scaled FP8 weights, per-row FP8 activations)" if w8a8 else "")
            + (" (packed-Q2 weights, group 128, bf16 activations)" if q2 else "")
            + (" fused gate+up weight" if fused else "")
            + (f" + LoRA rank {lora_rank} on gate, up, down" if lora_rank else "")
            + (" [warm: one weight replica, cache-resident]" if warm else ""))


def measure_ffn(name, steps, warmup, w4a4=False, m=None, fused=False, lora_rank=0, w8a8=False,
                q2=False, warm=False, ramp_s=RAMP_S):
    import torch

    import nvfp4_weight_dense_amd as nv
    import synthetic_inputs as si

    dev = torch.device("cuda:0")
    gen = si.fp8_workload if w8a8 else (si.q2_workload if q2 else si.workload)
    x, wg, wu, wd = gen(name, m=m)
    m, hidden = x.shape
    inter = wg.n
    wbytes = weight_bytes(wg) + weight_bytes(wu) + weight_bytes(wd)
    nrep = 1 if warm else max(1, math.ceil(REPLICA_BYTES / wbytes))
    xd = x.to(dev)
    out = torch.empty((m, hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    lp = None
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
    ms = _time_loop(lambda r: fn(xd, *r, out=out, stream=stream), reps, steps, warmup, stream,
                    ramp_s=ramp_s)
    # one more call on the first replica, kept for the oracle comparison
    fn(xd, *reps[0], out=out, stream=stream)
    torch.cuda.synchronize()
    flops = 6.0 * m * hidden * inter
    res = {
        "workload": _label(name, m, hidden, inter, w4a4, w8a8, q2, fused, lora_rank, warm),
        "m": m, "hidden": hidden, "inter": inter,
        "ms_per_step": ms,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "weight_gbs": wbytes / (ms * 1e-3) / 1e9,
        "weight_bytes": wbytes,
        "replicas": nrep,
    }
    res["hbm_frac"] = res["weight_gbs"] / HBM_PEAK_GBS
    res["mfma_frac"] = res["tflops"] / (FP8_PEAK_TFLOPS if w8a8 else BF16_PEAK_TFLOPS)
    check = dict(name=name, x=x, weights=(wg, wu, wd), y=out.cpu(), w4a4=w4a4, w8a8=w8a8, q2=q2,
                 lora=lora_rank, ms=ms, m=m)
    ctx = dict(x=xd, weights=reps, out=out, stream=stream, wbytes=wbytes, check=check)
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


def measure_mfma_peak():
    """Best of three runs of the register-only bf16 MFMA loop."""
    import torch

    import nvfp4_weight_dense_amd as nv

    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs, iters = 2 * cus, 20000
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    nv.nvfp4_probe_mfma_bf16(wgs, 2000, sink, stream)
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        nv.nvfp4_probe_mfma_bf16(wgs, iters, sink, stream)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end)
        best = ms if best is None else min(best, ms)
    flops = float(wgs) * 4 * iters * 4 * 32768
    return {
        "measured_tflops": flops / (best * 1e-3) / 1e12,
        "spec_tflops": BF16_PEAK_TFLOPS,
        "kernel": "v_mfma_f32_32x32x16_bf16, register operands, 4 independent chains per wave",
        "workgroups": wgs, "waves_per_workgroup": 4, "iters": iters, "ms": best,
    }


def measure_read_floor(sizes, steps, warmup):
    """HBM read rate of a launch that only streams: nvfp4_probe_read over
    each byte count in `sizes`, back to back on cold buffers (rotated so
    that their sum exceeds the caches), timed like the FFN.  This is what a
    single launch of that size reaches with nothing but loads -- ramp,
    latency and drain included -- the practical ceiling for the
    memory-bound launches beside the 8 TB/s of the specification."""
    import torch

    import nvfp4_weight_dense_amd as nv

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    top = max(sizes)
    top = (top + 15) // 16 * 16
    nrep = max(2, math.ceil(REPLICA_BYTES / top))
    # bytes 0x01: every 32-bit word is 0x01010101, and a lane folds sixteen
    # of them (or zeros) by xor, so the fold is 0 and never equals 0x5A5A5A5A
    bufs = [torch.full((top,), 1, dtype=torch.uint8, device=dev) for _ in range(nrep)]
    out = []
    for nb in sizes:
        nb16 = nb // 16 * 16
        ms = _time_loop(lambda b: nv.nvfp4_probe_read(b, nb16, 0x5A5A5A5A, sink, stream), bufs,
                        steps, warmup, stream)
        out.append({"bytes": nb16, "us": ms * 1e3, "gbs": nb16 / (ms * 1e-3) / 1e9})
    assert float(sink.abs().sum()) == 0.0
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "k_read_probe (nvfp4_probe_read): 256-lane workgroups, four 16-byte loads "
                      "in flight per lane, nothing else", "per_launch": out}


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


# launch patterns for the rocprofv3 counter passes: (workload, extra measure_ffn args)
KERNEL_RUNS = {
    "decode": ("decode", {}),
    "w4a4": ("w4a4", dict(m=1, w4a4=True)),
    "w8a8": ("w8a8", dict(m=1, w8a8=True)),
    "q2": ("decode", dict(m=1, q2=True)),
    "smallm": ("smallm", {}),
    "prefill": ("prefill", {}),
    "w4a4_64": ("w4a4", dict(m=64, w4a4=True)),
    "w4a4_512": ("w4a4", dict(m=512, w4a4=True)),
    "w8a8_64": ("w8a8", dict(m=64, w8a8=True)),
    "w8a8_512": ("w8a8", dict(m=512, w8a8=True)),
    "q2_prefill": ("prefill", dict(q2=True)),
    "q2_smallm": ("smallm", dict(q2=True)),
}


def traffic_run(steps, what="gemv"):
    """Launch pattern for the rocprofv3 counter passes: `steps` launches of
    the dominant kernel over rotating cold replicas (what="gemv"), `steps`
    whole FFNs of one workload (KERNEL_RUNS), `steps` runs of the MFMA
    probe (what="probe") or pairs of read-probe launches over the decode
    weight byte counts (what="read"); then `steps` plain device copies of COPY_BYTES,
    whose counter readings calibrate the memory counters against a
    transfer of known size.  No clock ramp: every dispatch is counted."""
    import torch

    import nvfp4_weight_dense_amd as nv

    dev = torch.device("cuda:0")
    if what == "probe":
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        sink = torch.zeros(256, dtype=torch.float32, device=dev)
        for _ in range(steps):
            nv.nvfp4_probe_mfma_bf16(2 * cus, 2000, sink)
        torch.cuda.synchronize()
    elif what == "read":
        # the read probe over the decode FFN's two weight byte counts, cold
        sink = torch.zeros(256, dtype=torch.float32, device=dev)
        sizes = (56623104, 28311552)
        bufs = [torch.full((sizes[0],), 1, dtype=torch.uint8, device=dev) for _ in range(8)]
        torch.cuda.synchronize()
        for i in range(steps):
            for nb in sizes:
                nv.nvfp4_probe_read(bufs[(2 * i + (nb == sizes[1])) % 8], nb, 0x5A5A5A5A, sink)
        torch.cuda.synchronize()
    else:
        if what == "gemv":
            _, ctx = measure_ffn("decode", 1, 0, ramp_s=0.0)
        else:
            name, kw = KERNEL_RUNS[what]
            _, ctx = measure_ffn(name, 1, 0, ramp_s=0.0, **kw)
        xd, reps, stream, out = ctx["x"], ctx["weights"], ctx["stream"], ctx["out"]
        chk = ctx["check"]
        act = torch.empty((xd.shape[0], reps[0][0].codes.shape[0]), dtype=torch.bfloat16,
                          device=xd.device)
        fn = (nv.dense_ffn_forward_w8a8 if chk["w8a8"] else nv.dense_ffn_forward_q2 if chk["q2"]
              else nv.dense_ffn_forward_w4a4 if chk["w4a4"] else nv.dense_ffn_forward)
        torch.cuda.synchronize()
        for i in range(steps):
            r = reps[i % len(reps)]
            if what == "gemv":
                nv.nvfp4_gate_up_silu_w4a16(xd, r[0], r[1], act=act, stream=stream)
            else:
                fn(xd, *r, out=out, stream=stream)
        torch.cuda.synchronize()
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_run": DOMINANT_KERNEL if what == "gemv" else what, "launches": steps,
                      "copy_bytes": COPY_BYTES, "source_hash": _kernel_source_hash()}),
          flush=True)


def _host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"cpu_count": os.cpu_count(), "usable_cores": usable, "model": model}


def _oracle_weights(check):
    import numpy as np
    import torch

    import oracle
    wg, wu, wd = check["weights"]
    if check["w8a8"]:
        return [oracle.Fp8Weight(w.codes.numpy(), w.scales.numpy()) for w in (wg, wu, wd)]
    if check["q2"]:
        return [oracle.Q2Weight(w.codes.numpy(), w.scales.view(torch.int16).numpy().view(np.uint16),
                                w.group) for w in (wg, wu, wd)]
    return [oracle.Weight(w.codes.numpy(), w.scales.numpy(), w.ts) for w in (wg, wu, wd)]


def oracle_check(check, threads, max_rows=2):
    """The oracle on a few rows of one workload: its time per row scaled to
    the workload's rows, and max |gpu - oracle| / rms(oracle) on those rows."""
    import numpy as np
    import torch

    import oracle
    import synthetic_inputs as si

    m = check["m"]
    rows = np.unique(np.array([0, m - 1][:max_rows]))
    xb = check["x"].view(torch.int16).numpy().view(np.uint16)[rows]
    ow = _oracle_weights(check)
    t0 = time.perf_counter()
    if check["w8a8"]:
        _, ye = oracle.dense_ffn_w8a8(xb, *ow, nthreads=threads)
    elif check["q2"]:
        _, ye = oracle.dense_ffn_q2(xb, *ow, nthreads=threads)
    elif check["lora"]:
        wg, wu, wd = check["weights"]
        inter, hidden = wg.n, wg.k
        pairs = []
        for n, k, which, scale in ((inter, hidden, 0, 2.0), (inter, hidden, 1, -1.5),
                                   (hidden, inter, 2, 0.5)):
            a, b = si.lora_pair(n, k, check["lora"], which=which)
            pairs.append(oracle.Lora(a.view(torch.int16).numpy().view(np.uint16),
                                     b.view(torch.int16).numpy().view(np.uint16), scale))
        _, ye = oracle.dense_ffn_lora(xb, *ow, *pairs, nthreads=threads)
    else:
        _, ye = oracle.dense_ffn(xb, *ow, w4a4=check["w4a4"], nthreads=threads)
    el = time.perf_counter() - t0
    got = check["y"][rows].double().numpy()
    rms = float(np.sqrt(np.mean(ye ** 2)))
    err = float(np.max(np.abs(got - ye))) / max(rms, 1e-300)
    est_s = el / len(rows) * m
    return {
        "oracle_rows": int(len(rows)),
        "oracle_s_per_ffn_est": est_s,
        "gpu_ms_per_ffn": check["ms"],
        "speedup_vs_oracle": est_s / (check["ms"] * 1e-3),
        "max_err_over_rms": err,
        "within_2e-2": bool(err <= 2e-2),
    }


def cpu_baseline(seconds=10.0, threads=None):
    import numpy as np

    import oracle
    import synthetic_inputs as si

    host = _host_cpu()
    if threads is None:
        threads = host["usable_cores"]
    x, wg, wu, wd = si.workload("decode")
    ow = [oracle.Weight(w.codes.numpy(), w.scales.numpy(), w.ts) for w in (wg, wu, wd)]
    xb = x.view(__import__("torch").int16).numpy().view(np.uint16)
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
        "threads": threads,
        "usable_cores": host["usable_cores"],
        "cpu_count": host["cpu_count"],
        "cpu_model": host["model"],
        "kind": "oracle",
        "sample": f"{reps} full decode FFNs (m=1, hidden=4096, inter=12288) in {el:.1f} s "
                  f"on {threads} threads",
        "ms_per_step": el / reps * 1e3,
    }


WORKLOAD_TABLE = (
    # name, steps divisor, w4a4, m, fused, lora rank, w8a8, q2, warm
    ("decode", 1, False, None, False, 0, False, True, False),
    ("smallm", 2, False, None, False, 0, False, True, False),
    ("prefill", 20, False, None, False, 0, False, True, False),
    ("decode", 1, False, None, True, 0, False, False, False),
    ("decode", 1, False, None, False, 16, False, False, False),
    ("smallm", 2, False, None, False, 0, False, False, False),
    ("prefill", 20, False, None, False, 0, False, False, False),
    ("decode", 1, False, None, False, 0, False, False, True),
    ("smallm", 2, False, None, False, 0, False, False, True),
    ("prefill", 20, False, None, False, 0, False, False, True),
    ("decode_tp8", 1, False, None, False, 0, False, False, False),
    ("prefill_tp8", 20, False, None, False, 0, False, False, False),
    ("w4a4", 2, True, 1, False, 0, False, False, False),
    ("w4a4", 2, True, 8, False, 0, False, False, False),
    ("w4a4", 2, True, 64, False, 0, False, False, False),
    ("w4a4", 20, True, 512, False, 0, False, False, False),
    ("w8a8", 2, False, 1, False, 0, True, False, False),
    ("w8a8", 2, False, 8, False, 0, True, False, False),
    ("w8a8", 2, False, 64, False, 0, True, False, False),
    ("w8a8", 20, False, 512, False, 0, True, False, False),
)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed calls before the timed ones (each workload first runs "
                         f"{RAMP_S} s of untimed calls for the GPU clock ramp)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-headline", action="store_true",
                    help="time only the decode workload (for profiling runs)")
    ap.add_argument("--only", default=None,
                    help="comma-separated workload names to time besides the headline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--traffic-run", nargs="?", const="gemv", default=None,
                    choices=("gemv", "probe", "read") + tuple(KERNEL_RUNS),
                    help="only launch the dominant kernel (or whole FFNs of one workload) "
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
    checks = [(head, ctx["check"])]
    roof = measure_dominant_kernel(ctx, args.steps, args.warmup)
    gu_bytes = weight_bytes(ctx["weights"][0][0]) + weight_bytes(ctx["weights"][0][1])
    d_bytes = weight_bytes(ctx["weights"][0][2])
    del ctx
    mfma = measure_mfma_peak()
    # the decode FFN's two launches, and one launch of all its bytes
    floor = measure_read_floor([gu_bytes, d_bytes, gu_bytes + d_bytes], args.steps, args.warmup)
    f_gu, f_d, f_all = floor["per_launch"]
    roof["read_floor_gbs"] = f_gu["gbs"]
    roof["frac_of_read_floor"] = roof["achieved"] / f_gu["gbs"]
    head["read_floor_two_launches_us"] = f_gu["us"] + f_d["us"]
    head["read_floor_one_launch_us"] = f_all["us"]
    head["frac_of_read_floor_two_launches"] = (f_gu["us"] + f_d["us"]) / (head["ms_per_step"] * 1e3)
    workloads = []
    only = None if args.only is None else set(args.only.split(","))
    invariance = {}
    if not args.only_headline:
        for name, div, w4a4, m, fused, rank, w8a8, q2, warm in WORKLOAD_TABLE:
            if only is not None and name not in only:
                continue
            steps = max(5 if div >= 20 else 20, args.steps // div)
            r, c = measure_ffn(name, steps, args.warmup, w4a4=w4a4, m=m, fused=fused,
                               lora_rank=rank, w8a8=w8a8, q2=q2, warm=warm)
            if r["m"] >= 512 or name in ("prefill", "prefill_tp8"):
                r["mfma_frac_measured_peak"] = r["tflops"] / mfma["measured_tflops"]
            if w4a4 or w8a8:
                invariance.setdefault("w4a4" if w4a4 else "w8a8", {})[r["m"]] = c["check"]["y"]
            checks.append((r, c["check"]))
            del c
            torch.cuda.empty_cache()
            workloads.append(r)
    # fixed formats: rows 0..m-1 at m < 512 equal the m = 512 run's rows bit for bit
    for fmt, ys in invariance.items():
        if 512 not in ys:
            continue
        for r in workloads:
            fmt_of = "w4a4" if r["workload"].endswith("w4a4") else ("w8a8" if "FP8" in r["workload"]
                                                                    else None)
            if fmt_of == fmt and r["m"] < 512:
                r["rows_bit_identical_to_m512"] = bool(torch.equal(
                    ys[r["m"]].view(torch.int16), ys[512][: r["m"]].view(torch.int16)))
    nv.nvfp4_release()
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args.cpu_seconds)
        per = []
        for r, chk in checks:
            rows = 1 if chk["m"] == 1 else 2
            entry = {"workload": r["workload"]}
            entry.update(oracle_check(chk, cpu["threads"], max_rows=rows))
            per.append(entry)
        cpu["per_config"] = per

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
            "ramp_s_before_warmup": RAMP_S,
        },
        "tflops": head["tflops"],
        "hbm_frac": head["hbm_frac"],
        "roofline": roof,
        "mfma_peak": mfma,
        "hbm_read_floor": floor,
        "read_floor_two_launches_us": head["read_floor_two_launches_us"],
        "read_floor_one_launch_us": head["read_floor_one_launch_us"],
        "frac_of_read_floor_two_launches": head["frac_of_read_floor_two_launches"],
        "cpu_baseline": cpu,
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
