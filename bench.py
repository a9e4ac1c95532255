#!/usr/bin/env python3
"""Benchmark: SSD forward tokens/s at Nemotron-Nano dims (seq 8192, bf16) on one MI355X.

One step = one whole forward pass (chunk cumsum, BMM, chunk state, state
passing, chunk scan -- or the single fused kernel) over one batch of synthetic
inputs already resident in HBM.  Prints ONE JSON line (rank 0).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload nemotron]
                    [--algo staged|fused|auto] [--no-cpu-baseline] [--input-dt]

--workload complex_434m prints the complex-A scan's own line (the Mamba-3-Lite
SSD Reference's 434M shape: three kernels; complex64 inputs, real output); the
default line carries a 20-step measurement of it in 'complex_fwd' (--no-complex
skips it), and the gated RMSNorm after the scan in 'gated_norm' (--no-norm).

--input-dt puts the step size on the input term as well (delta x (outer) B,
the discretised input of the Mamba-2 models); the default is the recurrence
as the pages write it.

Only one GPU is used: --gpus above 1 exits with a message.

Timing: W untimed steps, then K steps bracketed by torch.cuda.synchronize();
wall time over the K steps gives `value`.  Inside the same timed region every
kernel is bracketed by HIP events on the stream it runs on, which gives each
kernel's average duration; the dominant one is reported against its roofline
(algorithmic bytes per launch / average duration vs 8 TB/s HBM).

Cold: after the timed region, --cold-steps forwards are timed one by one with
HIP events, each preceded (outside the events) by a 512 MB write that evicts
the inputs from L2 and the 256 MB MALL; their median is reported as `cold`.

cpu_baseline: the fp64 oracle (C, OpenMP) on the host's cores over the same
workload, timed separately (a reported baseline, not the target).

--copy-calibration makes the program start with one 512 MiB device-to-device
copy, the reference transfer that HBM byte counters are scaled against.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3     # dense fp32 MFMA, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="nemotron")
    ap.add_argument("--seqlen", type=int, default=None,
                    help="override the workload's sequence length (e.g. a sweep over the "
                         "vLLM microbenchmark's 1k-64k tokens at granite dims)")
    ap.add_argument("--algo", default="auto", choices=["auto", "staged", "fused"])
    ap.add_argument("--state-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--out-dtype", default="bf16", choices=["f32", "bf16"])
    ap.add_argument("--layout", default="xbc", choices=["xbc", "contiguous"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--input-dt", action="store_true",
                    help="step size on the input term too (Mamba-2's discretised input)")
    ap.add_argument("--no-backward", dest="backward", action="store_false",
                    help="skip timing ssd_backward (by default it is timed with an upstream "
                         "gradient ~ N(0,1) and the forward+backward rate is reported in a "
                         "'fwd_bwd' object)")
    ap.add_argument("--backward", dest="backward", action="store_true",
                    help="time ssd_backward (the default)")
    ap.add_argument("--no-norm", dest="norm", action="store_false",
                    help="skip timing the gated RMSNorm after the scan (by default its forward "
                         "and backward are timed at the workload's shape in a 'gated_norm' "
                         "object)")
    ap.add_argument("--no-complex", dest="complex", action="store_false",
                    help="skip the complex-A forward at the SSD Reference's 434M shape (by "
                         "default timed for 20 steps in a 'complex_fwd' object)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle until this much CPU time has been spent (min 3 runs)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="event-timed forwards each preceded by a 512 MB cache flush")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="copy a 512 MiB device buffer once first (HBM counter calibration)")
    return ap.parse_args()


def stage_bytes(w, K, state_bytes, out_bytes, in_bytes=2, input_dt=False):
    """Algorithmic HBM bytes each kernel must move per launch (one forward).

    b*T tokens, H heads, P head dim, G groups, N state, C chunk, K chunk slots.
    Each input is read once, each output written once; CB is fp32 and only its
    causal half (s <= l) is written and read; the cumsum is fp32, and so are
    the per-position step sizes the staged path passes on with input_dt.
    """
    T = w.batch * w.seqlen
    H, P, G, N, C = w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk_size
    e = in_bytes
    x = T * H * P * e
    bc = T * G * N * e
    dt = T * H * e
    cs = 4 * K * H * C
    dtc = 4 * K * H * C if input_dt else 0
    cb = 4 * K * G * C * (C + 1) // 2
    st = K * H * P * N * state_bytes
    fin = 4 * (w.nseq or w.batch) * H * P * N
    z = x if w.has_z else 0
    out = T * H * P * out_bytes
    nseq = w.nseq or w.batch
    return {
        # cu_seqlens in; the chunk table (4-word header, 3 words per chunk,
        # first chunk per sequence) out
        "varlen_meta": 4 * (nseq + 1) + 4 * (4 + 3 * K + nseq + 1),
        "chunk_cumsum": dt + cs + dtc,
        "bmm_chunk": 2 * bc + cb,
        "chunk_state": x + bc + cs + dtc + st,
        "state_passing": 2 * st + 4 * K * H + fin,
        "chunk_scan": cb + x + bc + cs + dtc + st + z + out,
        "fused_fwd": x + 2 * bc + dt + z + out + fin,
    }


def stage_flops(w, K):
    """Useful matrix flops per launch (causal half only, no hi/lo second pass)."""
    H, P, G, N, C = w.nheads, w.headdim, w.ngroups, w.dstate, w.chunk_size
    f = {
        "varlen_meta": 0,
        "chunk_cumsum": 0,
        "bmm_chunk": K * G * C * (C + 1) * N,
        "chunk_state": 2 * K * H * C * P * N,
        "state_passing": 2 * K * H * P * N,
        "chunk_scan": 2 * K * H * C * N * P + K * H * C * (C + 1) * P,
    }
    f["fused_fwd"] = f["bmm_chunk"] + f["chunk_state"] + f["chunk_scan"]
    return f


KERNEL_SOURCES = {"chunk_cumsum": ("chunk_cumsum.hip", "stage_cumsum.hpp"),
                  "bmm_chunk": ("bmm_chunk.hip", "stage_bmm.hpp"),
                  "chunk_state": ("chunk_state.hip", "stage_state.hpp"),
                  "state_passing": ("state_passing.hip", "stage_passing.hpp"),
                  "chunk_scan": ("chunk_scan.hip", "stage_scan.hpp"),
                  "fused_fwd": ("fused_fwd.hip", "stage_varlen.hpp"),
                  "cx_chunk_state": ("complex_fwd.hip",),
                  "cx_state_passing": ("complex_fwd.hip",),
                  "cx_chunk_scan": ("complex_fwd.hip",)}


def measured_traffic(stage, key):
    """HBM bytes per launch from the committed counter summary, or None.

    profiles/hbm_traffic.json records, per configuration and kernel, the
    calibrated FETCH_SIZE + WRITE_SIZE bytes and a hash of the kernel's
    source; a kernel whose source changed since the counters were taken
    reports None.
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if stage not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(key, {}).get(stage)
    if not rec:
        return None
    csrc = os.path.join(ROOT, "mamba_ssd_chunked_scan_amd", "csrc")
    h = hashlib.sha256()
    for f in (*KERNEL_SOURCES[stage], "common.hpp", "kernels.hpp"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    if h.hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def cpu_baseline(w, inp, seconds):
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    times = []
    oracle.ssd_fwd(inp.x, inp.B, inp.C, inp.dt, inp.A, inp.dt_bias, inp.D, inp.z,
                   cu_seqlens=inp.cu_seqlens, threads=threads)  # warm-up (page-in)
    while len(times) < 3 or (sum(times) < seconds and len(times) < 1000):
        t0 = time.perf_counter()
        oracle.ssd_fwd(inp.x, inp.B, inp.C, inp.dt, inp.A, inp.dt_bias, inp.D, inp.z,
                       cu_seqlens=inp.cu_seqlens, threads=threads)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": w.tokens / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"the whole {w.name} workload ({w.tokens} tokens, all {w.nheads} heads), "
                       f"fp64 sequential recurrence, median of {len(times)} runs "
                       f"({sum(times):.1f} s) after 1 warm-up"),
            "seconds": t, "cpu": platform.processor() or platform.machine()}


def environment(torch, ssd):
    """Provenance of a measurement: device, compute units, software versions and the
    source revision when a git checkout is present."""
    import subprocess
    props = torch.cuda.get_device_properties(0)
    commit = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short", "HEAD"],
                           capture_output=True, text=True, timeout=5)
        commit = r.stdout.strip() or None
    except Exception:
        commit = None
    return {"gpu": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "hbm_GB": round(props.total_memory / 1e9, 1),
            "hip": torch.version.hip, "torch": torch.__version__,
            "libssd": ssd.lib().ssd_version().decode(), "commit": commit,
            "host_cpu": platform.processor() or platform.machine(),
            "host_cores": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested). "
              "The path would shard over heads/groups with no communication; see the design "
              "notes.", file=sys.stderr)
        sys.exit(2)
    import torch
    from mamba_ssd_chunked_scan_amd import ssd
    from mamba_ssd_chunked_scan_amd.inputs import COMPLEX_WORKLOADS, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.workload in COMPLEX_WORKLOADS:
        bench_complex(args, COMPLEX_WORKLOADS[args.workload])
        return
    w = WORKLOADS[args.workload]
    if args.seqlen is not None:
        import dataclasses
        w = dataclasses.replace(w, seqlen=args.seqlen)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    sdt = torch.float32 if args.state_dtype == "f32" else torch.bfloat16
    odt = torch.bfloat16 if args.out_dtype == "bf16" else torch.float32

    def up(a, dt=tdt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)

    if args.layout == "xbc":
        lead = inp.x.shape[:-2]
        H, P, G, N = w.nheads, w.headdim, w.ngroups, w.dstate
        buf = up(np.concatenate([inp.x.reshape(lead + (H * P,)), inp.B.reshape(lead + (G * N,)),
                                 inp.C.reshape(lead + (G * N,))], axis=-1))
        x = buf[..., :H * P].unflatten(-1, (H, P))
        B = buf[..., H * P:H * P + G * N].unflatten(-1, (G, N))
        C = buf[..., H * P + G * N:].unflatten(-1, (G, N))
    else:
        x, B, C = up(inp.x), up(inp.B), up(inp.C)
    dt, z = up(inp.dt), up(inp.z)
    A, bias = up(inp.A, torch.float32), up(inp.dt_bias, torch.float32)
    D = up(inp.D, torch.float32)
    cu = (torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
          if inp.cu_seqlens is not None else None)

    prob = ssd.problem_from(x, B, w.chunk_size, cu_seqlens=cu, state_dtype=sdt,
                            input_dt=args.input_dt)
    algo = args.algo
    if algo == "auto":
        # the single-pass forward where it applies (bf16 inputs, d_state <= 128),
        # the staged one otherwise
        algo = "fused" if (w.dtype == "bf16" and w.dstate <= 128) else "staged"
    K = prob.num_chunks()
    out = torch.empty(x.shape, dtype=odt, device=dev)
    nseq = prob.nseq if prob.packed else prob.batch
    fin = torch.empty((nseq, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device=dev)
    ws = torch.empty(max(prob.workspace_size(algo), 1), dtype=torch.uint8, device=dev)

    # stage buffers for the instrumented staged step (same kernels ssd_forward launches)
    cs = torch.empty((K, w.nheads, w.chunk_size), dtype=torch.float32, device=dev)
    dtc = torch.empty_like(cs) if args.input_dt else None
    cb = torch.empty((K, w.ngroups, w.chunk_size, w.chunk_size), dtype=torch.float32, device=dev)
    st = torch.empty((K, w.nheads, w.headdim, w.dstate), dtype=sdt, device=dev)
    if prob.packed:
        prob.chunk_meta = torch.empty(prob.meta_len(), dtype=torch.int32, device=dev)

    if algo == "staged":
        names = (["varlen_meta"] if prob.packed else []) + [
            "chunk_cumsum", "bmm_chunk", "chunk_state", "state_passing", "chunk_scan"]

        def launches():
            if prob.packed:
                yield "varlen_meta", lambda: ssd.ssd_varlen_chunk_meta(prob, prob.chunk_meta)
            yield "chunk_cumsum", lambda: ssd.ssd_chunk_cumsum(prob, dt, A, bias, cs, dtc)
            yield "bmm_chunk", lambda: ssd.ssd_bmm_chunk(prob, C, B, cb)
            yield "chunk_state", lambda: ssd.ssd_chunk_state(prob, x, B, cs, st, dt_chunk=dtc)
            yield "state_passing", lambda: ssd.ssd_state_passing(prob, st, cs, None, st, fin)
            yield "chunk_scan", lambda: ssd.ssd_chunk_scan(prob, cb, x, C, cs, st, D, z, out,
                                                           dt_chunk=dtc)
    else:
        names = ["fused_fwd"]

        def launches():
            yield "fused_fwd", lambda: ssd.ssd_forward(x, B, C, dt, A, bias, D, z, None, cu,
                                                       w.chunk_size, state_dtype=sdt, out=out,
                                                       final_states=fin, algo="fused",
                                                       workspace=ws, input_dt=args.input_dt)

    def step(events=None):
        for name, fn in launches():
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                events.setdefault(name, []).append((e0, e1))
            else:
                fn()

    # correctness smoke of the timed configuration against ssd_forward (same kernels)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_kernel_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in events[n]])) for n in names}

    # cold: a 512 MB write before each forward evicts L2 and the MALL
    cold_ms = []
    if args.cold_steps > 0:
        flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        for _ in range(args.cold_steps):
            flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _name, fn in launches():
                fn()
            e1.record()
            torch.cuda.synchronize()
            cold_ms.append(e0.elapsed_time(e1))
        del flush
    ms_per_step = wall * 1e3 / args.steps
    tokens = w.tokens
    value = tokens * args.steps / wall

    # host submission: the time one whole forward call takes to return on the host
    # (every launch is asynchronous), each timed on an idle queue
    submit_us = []
    for _ in range(20):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for _name, fn in launches():
            fn()
        submit_us.append((time.perf_counter() - h0) * 1e6)
    torch.cuda.synchronize()

    sbytes = 4 if sdt == torch.float32 else 2
    obytes = 2 if odt == torch.bfloat16 else 4
    ibytes = 2 if w.dtype == "bf16" else 4
    nb = stage_bytes(w, K, sbytes, obytes, ibytes, args.input_dt)
    nf = stage_flops(w, K)
    dom = max((n for n in names if n in nb), key=lambda n: per_kernel_ms[n])
    achieved = nb[dom] / (per_kernel_ms[dom] * 1e-3) / 1e9
    stages = {n: {"ms": round(per_kernel_ms[n], 5),
                  "GBps": (round(nb[n] / (per_kernel_ms[n] * 1e-3) / 1e9, 1) if n in nb else None),
                  "hbm_frac": (round(nb[n] / (per_kernel_ms[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                               if n in nb else None),
                  "mfma_TFLOPs": (round(nf[n] / (per_kernel_ms[n] * 1e-3) / 1e12, 1)
                                  if nf.get(n) else None)}
              for n in names}
    roof_time_ms = sum(nb[n] for n in names if n in nb) / (HBM_PEAK_GBS * 1e9) * 1e3

    traffic_key = (f"{w.name}_{algo}_{args.state_dtype}state_{args.out_dtype}out_{args.layout}"
                   + ("_inputdt" if args.input_dt else ""))
    result = {
        "metric": "SSD fwd tokens/s at Nemotron-Nano dims, seq 8192 bf16; % of stage roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: SSD forward, batch {w.batch}, seq {w.seqlen}, "
                        f"{w.nheads} heads x {w.headdim}, d_state {w.dstate}, "
                        f"{w.ngroups} groups, chunk {w.chunk_size}"
                        + (f", {w.nseq} packed sequences" if w.nseq else "")
                        + (", D" if w.has_D else "") + (", z gate" if w.has_z else "")
                        + (", step size on the input term" if args.input_dt else ""),
            "global_batch": w.batch, "seq_len": w.seqlen, "parallelism": "none (1 GPU)",
            "algo": algo, "state_dtype": args.state_dtype, "out_dtype": args.out_dtype,
            "layout": args.layout, "input_dt": bool(args.input_dt),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom, traffic_key),
            "bytes_per_launch": nb[dom],
            "avg_launch_ms": round(per_kernel_ms[dom], 5),
        },
        "stages": stages,
        "path_roofline_frac": round(roof_time_ms / ms_per_step, 4),
        "host_submit_us": round(float(np.median(submit_us)), 1),
        "cold": ({"ms_median": round(float(np.median(cold_ms)), 5),
                  "value": round(tokens / (float(np.median(cold_ms)) * 1e-3), 1),
                  "steps": len(cold_ms),
                  "note": "median of event-timed forwards, each after a 512 MB cache flush"}
                 if cold_ms else None),
        "gpu": torch.cuda.get_device_name(0),
        "env": environment(torch, ssd),
    }
    if args.backward:
        result["fwd_bwd"] = time_backward(args, w, ssd, x, B, C, dt, A, bias, D, z, cu,
                                          ms_per_step)
    if args.norm:
        result["gated_norm"] = time_norm(args, w, ssd, dev)
    if args.complex:
        from mamba_ssd_chunked_scan_amd.inputs import COMPLEX_WORKLOADS
        cx = measure_complex(args, COMPLEX_WORKLOADS["complex_434m"], steps=20,
                             warmup=min(args.warmup, 5))
        result["complex_fwd"] = {k: cx[k] for k in ("metric", "value", "unit", "ms_per_step",
                                                    "steps", "config", "roofline", "stages",
                                                    "path_roofline_frac")}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def time_norm(args, w, ssd, dev):
    """HIP-event times of the gated RMSNorm forward and backward at the workload's
    output shape (bf16 y, z, dout; fp32 dy, dz; norm groups of H P / G channels,
    Mamba-2's d_inner / ngroups), against their algorithmic bytes."""
    import torch
    H, P = w.nheads, w.headdim
    gs = H * P // w.ngroups
    shape = (w.batch, w.seqlen, H, P)
    g = torch.Generator(device=dev).manual_seed(5)
    y = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    z = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    dout = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    wt = torch.ones(H * P, device=dev)
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    ntok = w.batch * w.seqlen
    el = ntok * H * P
    fwd_bytes = 3 * 2 * el + 4 * H * P
    ntile = -(-ntok // 64)
    bwd_bytes = 3 * 2 * el + 2 * 4 * el + 4 * H * P * 2 + 2 * 4 * ntile * H * P

    dy = torch.empty(shape, dtype=torch.float32, device=dev)
    dz = torch.empty(shape, dtype=torch.float32, device=dev)
    dw = torch.empty(H * P, dtype=torch.float32, device=dev)
    ws = torch.empty(max(ssd.gated_rmsnorm_bwd_workspace_size(y, gs), 1), dtype=torch.uint8,
                     device=dev)

    def timed(fn, n):
        # n calls back to back between two events: the queue stays ahead of the GPU
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    fwd = lambda: ssd.ssd_gated_rmsnorm_fwd(y, z, wt, gs, out=out)
    bwd = lambda: ssd.ssd_gated_rmsnorm_bwd(y, z, wt, dout, gs, workspace=ws, dy=dy, dz=dz, dw=dw)
    for _ in range(3):
        fwd()
        bwd()
    torch.cuda.synchronize()
    n = max(10, args.steps // 2)
    fm, bm = timed(fwd, n), timed(bwd, n)
    return {"group_size": gs, "fwd_ms": round(fm, 5), "bwd_ms": round(bm, 5),
            "fwd_GBps": round(fwd_bytes / (fm * 1e-3) / 1e9, 1),
            "bwd_GBps": round(bwd_bytes / (bm * 1e-3) / 1e9, 1),
            "fwd_hbm_frac": round(fwd_bytes / (fm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bwd_hbm_frac": round(bwd_bytes / (bm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fwd_bytes": fwd_bytes, "bwd_bytes": bwd_bytes,
            "calls": n,
            "note": "average over calls issued back to back between two HIP events; the "
                    "backward includes its weight-gradient partials and their reduction"}


def time_backward(args, w, ssd, x, B, C, dt, A, bias, D, z, cu, fwd_ms):
    """HIP-event time of ssd_backward (all gradients) on the same inputs, with
    an upstream gradient drawn from N(0, 1); the forward+backward rate adds
    the forward step time measured above."""
    import torch
    g = torch.Generator(device=x.device).manual_seed(4)
    dout = torch.randn(x.shape, generator=g, device=x.device, dtype=torch.float32)
    prob = ssd.problem_from(x, B, w.chunk_size, cu_seqlens=cu, input_dt=args.input_dt)
    ws = torch.empty(prob.backward_workspace_size(), dtype=torch.uint8, device=x.device)

    def bwd():
        return ssd.ssd_backward(x, B, C, dt, A, dout, dt_bias=bias, D=D, z=z, cu_seqlens=cu,
                                chunk_size=w.chunk_size, workspace=ws, input_dt=args.input_dt)

    for _ in range(max(2, args.warmup // 5)):
        bwd()
    torch.cuda.synchronize()
    times = []
    for _ in range(max(5, args.steps // 5)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        bwd()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    bms = float(np.median(times))
    # the backward's algorithmic bytes: read x, B, C, dt, z (input dtype) and dout
    # (fp32); write dx, dB, dC, ddt, dz (fp32); per-head vectors are negligible
    tok = w.batch * w.seqlen
    H, P, G, N = w.nheads, w.headdim, w.ngroups, w.dstate
    e = 2 if w.dtype == "bf16" else 4
    zb = tok * H * P if w.has_z else 0
    alg = (e * (tok * H * P + 2 * tok * G * N + tok * H + zb) + 4 * tok * H * P
           + 4 * (tok * H * P + 2 * tok * G * N + tok * H + zb))
    return {"bwd_ms": round(bms, 5), "fwd_ms": round(fwd_ms, 5),
            "bwd_algorithmic_bytes": alg,
            "bwd_hbm_frac": round(alg / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fwd_bwd_ms": round(bms + fwd_ms, 5),
            "tokens_per_s": round(w.tokens / ((bms + fwd_ms) * 1e-3), 1),
            "workspace_MB": round(ws.numel() / 1e6, 1), "steps": len(times),
            "note": "median of event-timed backward calls, plus the "
                    "timed forward step"}


def complex_stage_model(w):
    """Algorithmic HBM bytes and useful matrix flops per launch of the three
    complex-A kernels (complex64 = 8 bytes; a complex multiply-add is 8 real
    flops, one whose imaginary part is not needed 4).  Each input is read once,
    each output written once; C.B^T and the intra-chunk product count their
    causal half only; the output is the real part (float32)."""
    b, T, H, P, N, C = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk_size
    nc = -(-T // C)
    K = b * nc
    tok = b * T
    x, bc, dt = tok * H * P * 8, tok * H * N * 8, tok * H * 4
    st, lam, fin, out = K * H * P * N * 8, K * H * 4, b * H * P * N * 8, tok * H * P * 4
    tri = C * (C + 1) // 2
    nb = {"cx_chunk_state": x + bc + dt + st + lam,
          "cx_state_passing": 2 * st + lam + fin,
          "cx_chunk_scan": x + 2 * bc + dt + st + out}
    nf = {"cx_chunk_state": 8 * K * H * C * P * N,
          "cx_state_passing": 8 * K * H * P * N,
          "cx_chunk_scan": K * H * (8 * tri * N + 4 * tri * P + 4 * C * N * P)}
    return nb, nf


def bench_complex(args, w):
    """Print the complex-A forward's own JSON line (bench.py --workload complex_434m)."""
    result = measure_complex(args, w)
    if not args.no_cpu_baseline:
        from mamba_ssd_chunked_scan_amd.inputs import make_complex_inputs
        result["cpu_baseline"] = cpu_baseline_complex(w, make_complex_inputs(w),
                                                      args.cpu_seconds)
    print(json.dumps(result), flush=True)


def measure_complex(args, w, steps=None, warmup=None):
    """The complex-A forward: ssd_complex_chunk_state, ssd_complex_state_passing,
    ssd_complex_chunk_scan (what ssd_complex_forward launches), each bracketed
    by HIP events on the stream it runs on.  Returns the result dict."""
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    import torch
    from mamba_ssd_chunked_scan_amd import ssd
    from mamba_ssd_chunked_scan_amd.inputs import make_complex_inputs

    inp = make_complex_inputs(w)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x, B, C, dt, A = up(inp.x), up(inp.B), up(inp.C), up(inp.dt), up(inp.A)
    h0 = up(inp.h0) if inp.h0 is not None else None
    prob = ssd.ComplexProblem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk_size)
    nc = -(-w.seqlen // w.chunk_size)
    st = torch.empty((w.batch * nc, w.nheads, w.headdim, w.dstate), dtype=torch.complex64,
                     device=dev)
    lam = torch.empty((w.nheads, w.batch * nc), dtype=torch.float32, device=dev)
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.complex64,
                      device=dev)
    out = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim), dtype=torch.float32, device=dev)
    names = ["cx_chunk_state", "cx_state_passing", "cx_chunk_scan"]
    calls = {
        "cx_chunk_state": lambda: ssd.ssd_complex_chunk_state(prob, x, B, dt, A, st, lam),
        "cx_state_passing": lambda: ssd.ssd_complex_state_passing(prob, A, lam, st, h0, fin),
        "cx_chunk_scan": lambda: ssd.ssd_complex_chunk_scan(prob, x, B, C, dt, A, st, out),
    }

    def step(events=None):
        for n in names:
            if events is None:
                calls[n]()
                continue
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            calls[n]()
            e1.record()
            events.setdefault(n, []).append((e0, e1))

    for _ in range(warmup):
        step()
    # the stage sequence is exactly ssd_complex_forward (one more untimed step, so
    # that the check also holds with no warm-up)
    step()
    ref_out, ref_fin = ssd.ssd_complex_forward(x, B, C, dt, A, initial_states=h0,
                                               chunk_size=w.chunk_size)
    torch.cuda.synchronize()
    if not (torch.equal(ref_out, out) and torch.equal(ref_fin, fin)):
        raise RuntimeError("stage sequence differs from ssd_complex_forward")
    events = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in events[n]])) for n in names}
    ms_per_step = wall * 1e3 / steps
    nb, nf = complex_stage_model(w)

    def roof(n):
        t_hbm = nb[n] / (HBM_PEAK_GBS * 1e9)
        t_mfma = nf[n] / (FP32_PEAK_TFLOPS * 1e12)
        return ("hbm", t_hbm) if t_hbm >= t_mfma else ("mfma", t_mfma)

    dom = max(names, key=lambda n: per_ms[n])
    bound, _ = roof(dom)
    if bound == "hbm":
        achieved, peak, unit = nb[dom] / (per_ms[dom] * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
    else:
        achieved, peak, unit = nf[dom] / (per_ms[dom] * 1e-3) / 1e12, FP32_PEAK_TFLOPS, "TFLOP/s"
    stages = {n: {"ms": round(per_ms[n], 5),
                  "GBps": round(nb[n] / (per_ms[n] * 1e-3) / 1e9, 1),
                  "fp32_mfma_TFLOPs": round(nf[n] / (per_ms[n] * 1e-3) / 1e12, 1),
                  "bound": roof(n)[0],
                  "roofline_frac": round(roof(n)[1] / (per_ms[n] * 1e-3), 4)}
              for n in names}
    roof_ms = sum(roof(n)[1] for n in names) * 1e3
    result = {
        "metric": "complex-A SSD fwd tokens/s (Mamba-3-Lite SSD Reference, 434M shape)",
        "value": round(w.tokens * steps / wall, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: complex-A SSD forward, batch {w.batch}, seq "
                               f"{w.seqlen}, {w.nheads} heads x {w.headdim}, d_state {w.dstate}, "
                               f"chunk {w.chunk_size}, complex64 x/B/C/A, float32 dt, "
                               "real output",
                   "global_batch": w.batch, "seq_len": w.seqlen,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": bound, "kernel": dom, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(dom, w.name), "bytes_per_launch": nb[dom],
                     "flops_per_launch": nf[dom],
                     "avg_launch_ms": round(per_ms[dom], 5)},
        "stages": stages,
        "path_roofline_frac": round(roof_ms / ms_per_step, 4),
        "gpu": torch.cuda.get_device_name(0),
        "env": environment(torch, ssd),
    }
    del x, B, C, dt, A, st, lam, fin, out, ref_out, ref_fin
    return result


def cpu_baseline_complex(w, inp, seconds):
    """The fp64 complex oracle on batch row 0 (all heads, all tokens), repeated
    for about `seconds`; tokens/s of that sample."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    sl = lambda a: None if a is None else a[:1]
    args = (sl(inp.x), sl(inp.B), sl(inp.C), sl(inp.dt), inp.A)
    oracle.ssd_complex_fwd(*args, initial_states=sl(inp.h0), threads=threads)
    times = []
    while len(times) < 3 or (sum(times) < seconds and len(times) < 1000):
        t0 = time.perf_counter()
        oracle.ssd_complex_fwd(*args, initial_states=sl(inp.h0), threads=threads)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": w.seqlen / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"batch row 0 of {w.name} ({w.seqlen} tokens, all {w.nheads} heads), "
                       f"fp64 sequential complex recurrence, median of {len(times)} runs "
                       f"({sum(times):.1f} s) after 1 warm-up"),
            "seconds": t, "cpu": platform.processor() or platform.machine()}


if __name__ == "__main__":
    main()
