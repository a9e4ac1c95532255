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

Timing: W untimed steps, then K timed steps bracketed by torch.cuda.synchronize().
Each timed step is preceded, outside its events, by a 512 MB write that evicts
the inputs from L2 and the 256 MB MALL (they stay resident in HBM); the step
and each launch in it are bracketed by HIP events on the stream they run on.
`value` and `ms_per_step` come from the median step (cold); the same K steps
back to back without the flush are reported as `warm`.  The dominant launch is
reported against its roofline (algorithmic bytes per launch / median cold
duration vs 8 TB/s HBM, and vs the achievable bandwidth of a 1 GiB copy
measured in the same run: `measured_peaks`).  The fused forward is one call of
three launches (range aggregates, their carry-ins, then outputs); its call is the
timed unit.

'configs' carries the other workloads (Granite dims, the packed batch, long
context fused and staged with fp32 / bf16 states, staged Nemotron-Nano with
both state dtypes), each cold and warm; 'gated_norm_fused' the forward with
the gated RMSNorm fused in against the two calls it replaces.

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
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the other workloads (Granite, packed, long context, staged "
                         "state dtypes) reported in a 'configs' object")
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


def measure_peaks(torch, dev):
    """Achievable peaks on this device: HBM bandwidth of a 1 GiB device-to-device
    copy (read + write bytes / time) and the dense bf16 matrix rate of an
    8192^3 GEMM through torch (hipBLASLt).  Medians of 10 event-timed runs."""
    src = torch.ones(2**28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)

    def med(fn, n=10):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    copy_ms = med(lambda: dst.copy_(src))
    gemm_ms = med(lambda: torch.matmul(a, b))
    res = {"hbm_copy_GBps": round(2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1),
           "bf16_gemm_TFLOPs": round(2 * 8192**3 / (gemm_ms * 1e-3) / 1e12, 1),
           "note": "1 GiB device-to-device copy (read + write bytes); 8192^3 bf16 GEMM "
                   "(torch.matmul); medians of 10 event-timed runs"}
    del src, dst, a, b
    return res


class Forward:
    """One forward configuration: inputs resident in HBM, preallocated outputs and
    workspace, and the launches ssd_forward makes (the staged path's five stage
    calls one by one, so each can be bracketed by events; the fused path as its
    one call)."""

    def __init__(self, torch, ssd, w, algo, state_dtype="f32", out_dtype="bf16", layout="xbc",
                 input_dt=False, dev=None):
        from mamba_ssd_chunked_scan_amd.inputs import make_inputs
        self.w, self.algo, self.state_dtype, self.out_dtype = w, algo, state_dtype, out_dtype
        self.input_dt = input_dt
        dev = dev or torch.device("cuda:0")
        inp = self.inp = make_inputs(w)
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        sdt = torch.float32 if state_dtype == "f32" else torch.bfloat16
        odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32

        def up(a, dt=tdt):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)

        if layout == "xbc":
            lead = inp.x.shape[:-2]
            H, P, G, N = w.nheads, w.headdim, w.ngroups, w.dstate
            buf = up(np.concatenate([inp.x.reshape(lead + (H * P,)),
                                     inp.B.reshape(lead + (G * N,)),
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
        self.t = dict(x=x, B=B, C=C, dt=dt, z=z, A=A, bias=bias, D=D, cu=cu)
        prob = self.prob = ssd.problem_from(x, B, w.chunk_size, cu_seqlens=cu, state_dtype=sdt,
                                            input_dt=input_dt)
        K = self.K = prob.num_chunks()
        out = self.out = torch.empty(x.shape, dtype=odt, device=dev)
        nseq = prob.nseq if prob.packed else prob.batch
        fin = self.fin = torch.empty((nseq, w.nheads, w.headdim, w.dstate), dtype=torch.float32,
                                     device=dev)
        self.ws = ws = torch.empty(max(prob.workspace_size(algo), 1), dtype=torch.uint8,
                                   device=dev)
        if algo == "staged":
            cs = torch.empty((K, w.nheads, w.chunk_size), dtype=torch.float32, device=dev)
            dtc = torch.empty_like(cs) if input_dt else None
            cb = torch.empty((K, w.ngroups, w.chunk_size, w.chunk_size), dtype=torch.float32,
                             device=dev)
            st = torch.empty((K, w.nheads, w.headdim, w.dstate), dtype=sdt, device=dev)
            if prob.packed:
                prob.chunk_meta = torch.empty(prob.meta_len(), dtype=torch.int32, device=dev)
            self.names = (["varlen_meta"] if prob.packed else []) + [
                "chunk_cumsum", "bmm_chunk", "chunk_state", "state_passing", "chunk_scan"]
            calls = {
                "varlen_meta": lambda: ssd.ssd_varlen_chunk_meta(prob, prob.chunk_meta),
                "chunk_cumsum": lambda: ssd.ssd_chunk_cumsum(prob, dt, A, bias, cs, dtc),
                "bmm_chunk": lambda: ssd.ssd_bmm_chunk(prob, C, B, cb),
                "chunk_state": lambda: ssd.ssd_chunk_state(prob, x, B, cs, st, dt_chunk=dtc),
                "state_passing": lambda: ssd.ssd_state_passing(prob, st, cs, None, st, fin),
                "chunk_scan": lambda: ssd.ssd_chunk_scan(prob, cb, x, C, cs, st, D, z, out,
                                                         dt_chunk=dtc),
            }
            self.calls = [(n, calls[n]) for n in self.names]
        else:
            self.names = ["fused_fwd"]
            self.calls = [("fused_fwd", lambda: ssd.ssd_forward(
                x, B, C, dt, A, bias, D, z, None, cu, w.chunk_size, state_dtype=sdt, out=out,
                final_states=fin, algo="fused", workspace=ws, input_dt=input_dt))]
        sb = 4 if state_dtype == "f32" else 2
        ob = 2 if out_dtype == "bf16" else 4
        ib = 2 if w.dtype == "bf16" else 4
        self.nb = stage_bytes(w, K, sb, ob, ib, input_dt)
        self.nf = stage_flops(w, K)
        self.path_bytes = sum(self.nb[n] for n in self.names)

    def run(self, torch, steps, flush=None):
        """`steps` forwards; each launch bracketed by HIP events, and the whole step
        too.  With `flush` (a large device buffer), every step is preceded, outside
        the events, by a write of it.  Returns (per-launch ms lists, step ms list)."""
        per = {n: [] for n in self.names}
        step_ms = []
        for _ in range(steps):
            if flush is not None:
                flush.fill_(1.0)
            evs = []
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record()
            for n, fn in self.calls:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                evs.append((n, e0, e1))
            s1.record()
            torch.cuda.synchronize()
            for n, e0, e1 in evs:
                per[n].append(e0.elapsed_time(e1))
            step_ms.append(s0.elapsed_time(s1))
        return per, step_ms

    def summary(self, torch, steps, warmup, flush):
        for _ in range(warmup):
            for _n, fn in self.calls:
                fn()
        torch.cuda.synchronize()
        cper, cstep = self.run(torch, steps, flush)
        wper, wstep = self.run(torch, steps, None)
        med = lambda v: float(np.median(v))
        cold, warm = med(cstep), med(wstep)
        tok = self.w.tokens
        res = {"algo": self.algo, "state_dtype": self.state_dtype, "out_dtype": self.out_dtype,
               "cold_ms": round(cold, 5), "warm_ms": round(warm, 5),
               "tokens_per_s": round(tok / (cold * 1e-3), 1),
               "warm_tokens_per_s": round(tok / (warm * 1e-3), 1),
               "algorithmic_bytes": self.path_bytes,
               "hbm_frac": round(self.path_bytes / (cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if len(self.names) > 1:
            res["stages_cold_ms"] = {n: round(med(cper[n]), 5) for n in self.names}
        return res, cper, wper, cstep, wstep


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested). "
              "The path would shard over heads/groups with no communication; see the design "
              "notes.", file=sys.stderr)
        sys.exit(2)
    import torch
    from mamba_ssd_chunked_scan_amd import ssd
    from mamba_ssd_chunked_scan_amd.inputs import COMPLEX_WORKLOADS, WORKLOADS

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
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(512 * 2**20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    algo = args.algo
    if algo == "auto":
        # the single-pass forward where it applies (bf16 inputs, d_state <= 128),
        # the staged one otherwise
        algo = "fused" if (w.dtype == "bf16" and w.dstate <= 128) else "staged"
    fw = Forward(torch, ssd, w, algo, args.state_dtype, args.out_dtype, args.layout,
                 args.input_dt, dev)
    # a 512 MB write before each cold step evicts the inputs from L2 and the 256 MB MALL
    flush = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)

    # warm-up, then K timed steps (each after a flush, outside the events),
    # bracketed by synchronisation; then K warm steps back to back
    for _ in range(args.warmup):
        for _n, fn in fw.calls:
            fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cper, cstep = fw.run(torch, args.steps, flush)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    wper, wstep = fw.run(torch, args.steps, None)
    med = lambda v: float(np.median(v))
    cold_ms, warm_ms = med(cstep), med(wstep)
    per_cold = {n: med(cper[n]) for n in fw.names}
    per_warm = {n: med(wper[n]) for n in fw.names}
    tokens = w.tokens
    value = tokens / (cold_ms * 1e-3)

    # host submission: the time one whole forward call takes to return on the host
    # (every launch is asynchronous), each timed on an idle queue
    submit_us = []
    for _ in range(20):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for _n, fn in fw.calls:
            fn()
        submit_us.append((time.perf_counter() - h0) * 1e6)
    torch.cuda.synchronize()

    peaks = measure_peaks(torch, dev)
    nb, nf = fw.nb, fw.nf
    dom = max((n for n in fw.names if n in nb), key=lambda n: per_cold[n])
    achieved = nb[dom] / (per_cold[dom] * 1e-3) / 1e9
    stages = {n: {"cold_ms": round(per_cold[n], 5), "warm_ms": round(per_warm[n], 5),
                  "GBps": (round(nb[n] / (per_cold[n] * 1e-3) / 1e9, 1) if n in nb else None),
                  "hbm_frac": (round(nb[n] / (per_cold[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                               if n in nb else None),
                  "mfma_TFLOPs": (round(nf[n] / (per_cold[n] * 1e-3) / 1e12, 1)
                                  if nf.get(n) else None)}
              for n in fw.names}
    roof_time_ms = fw.path_bytes / (HBM_PEAK_GBS * 1e9) * 1e3

    traffic_key = (f"{w.name}_{algo}_{args.state_dtype}state_{args.out_dtype}out_{args.layout}"
                   + ("_inputdt" if args.input_dt else ""))
    result = {
        "metric": "SSD fwd tokens/s at Nemotron-Nano dims, seq 8192 bf16; % of stage roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "timing": ("value and ms_per_step: median of K event-timed forwards, each preceded "
                   "(outside the events) by a 512 MB write that evicts L2 and the MALL; the "
                   "inputs stay resident in HBM.  'warm': the same K forwards back to back "
                   f"without the flush.  Wall time of the K cold steps: {wall:.3f} s"),
        "warm": {"ms_median": round(warm_ms, 5), "value": round(tokens / (warm_ms * 1e-3), 1)},
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
            "kernel": dom + (" (the call: range-aggregate, carry and output launches)"
                             if dom == "fused_fwd" else ""),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom, traffic_key),
            "bytes_per_launch": nb[dom],
            "avg_launch_ms": round(per_cold[dom], 5),
            "achievable_peak": peaks["hbm_copy_GBps"],
            "frac_of_achievable": round(achieved / peaks["hbm_copy_GBps"], 4),
        },
        "stages": stages,
        "path_roofline_frac": round(roof_time_ms / cold_ms, 4),
        "measured_peaks": peaks,
        "mfma": {"useful_TFLOPs": round(nf[dom] / (per_cold[dom] * 1e-3) / 1e12, 1),
                 "frac_of_published": round(nf[dom] / (per_cold[dom] * 1e-3) / 1e12
                                            / BF16_PEAK_TFLOPS, 4),
                 "frac_of_achievable": round(nf[dom] / (per_cold[dom] * 1e-3) / 1e12
                                             / peaks["bf16_gemm_TFLOPs"], 4),
                 "note": "useful causal matrix flops (no hi/lo second pass); a diagnostic: "
                         "the path is bound by HBM bytes at these shapes"} if nf.get(dom) else None,
        "host_submit_us": round(float(np.median(submit_us)), 1),
        "gpu": torch.cuda.get_device_name(0),
        "env": environment(torch, ssd),
    }
    del fw
    if args.configs and args.workload == "nemotron" and args.seqlen is None:
        result["configs"] = other_configs(args, torch, ssd, flush)
    if args.norm:
        result["gated_norm"] = time_norm(args, w, ssd, dev)
        if w.dtype == "bf16" and w.dstate <= 128 and w.headdim % 64 == 0:
            result["gated_norm_fused"] = time_norm_fused(args, w, ssd, torch, flush)
    if args.backward:
        fw2 = Forward(torch, ssd, w, algo, args.state_dtype, args.out_dtype, args.layout,
                      args.input_dt, dev)
        t = fw2.t
        result["fwd_bwd"] = time_backward(args, w, ssd, t["x"], t["B"], t["C"], t["dt"], t["A"],
                                          t["bias"], t["D"], t["z"], t["cu"], cold_ms)
        del fw2
    if args.complex:
        from mamba_ssd_chunked_scan_amd.inputs import COMPLEX_WORKLOADS
        cx = measure_complex(args, COMPLEX_WORKLOADS["complex_434m"], steps=20,
                             warmup=min(args.warmup, 5))
        result["complex_fwd"] = {k: cx[k] for k in ("metric", "value", "unit", "ms_per_step",
                                                    "steps", "config", "roofline", "stages",
                                                    "path_roofline_frac")}
    if not args.no_cpu_baseline:
        from mamba_ssd_chunked_scan_amd.inputs import make_inputs
        result["cpu_baseline"] = cpu_baseline(w, make_inputs(w), args.cpu_seconds)
    print(json.dumps(result), flush=True)


def other_configs(args, torch, ssd, flush):
    """The other workloads the pages time, each cold (median of 10 forwards after a
    flush) and warm: Granite-style (vLLM PR 27299's SSD microbenchmark dims, seq
    4096), the packed 8-sequence Nemotron-Nano batch, long context (seq 65536,
    chunk 256; fused, and staged with fp32 and bf16 per-chunk states), and the
    staged Nemotron-Nano path with both state dtypes."""
    from mamba_ssd_chunked_scan_amd.inputs import WORKLOADS
    out = {}
    for key, name, algo, sd in [("granite_fused", "granite", "fused", "f32"),
                                ("nemotron_varlen_fused", "nemotron_varlen", "fused", "f32"),
                                ("longctx_fused", "longctx", "fused", "f32"),
                                ("longctx_staged_f32state", "longctx", "staged", "f32"),
                                ("longctx_staged_bf16state", "longctx", "staged", "bf16"),
                                ("nemotron_staged_f32state", "nemotron", "staged", "f32"),
                                ("nemotron_staged_bf16state", "nemotron", "staged", "bf16")]:
        w = WORKLOADS[name]
        fw = Forward(torch, ssd, w, algo, sd, "bf16", "xbc", False)
        res = fw.summary(torch, 10, 3, flush)[0]
        res["workload"] = (f"{w.name}: batch {w.batch}, seq {w.seqlen}, {w.nheads} heads x "
                           f"{w.headdim}, d_state {w.dstate}, {w.ngroups} groups, chunk "
                           f"{w.chunk_size}" + (f", {w.nseq} packed sequences" if w.nseq else ""))
        out[key] = res
        del fw
        torch.cuda.empty_cache()
    return out


def time_norm_fused(args, w, ssd, torch, flush):
    """The forward with the gated RMSNorm fused in (ssd_forward_gated_norm, groups of
    H P / G channels) against the two calls it replaces (ssd_forward without the
    gate, then ssd_gated_rmsnorm_fwd), cold (each after a flush) and warm."""
    fw = Forward(torch, ssd, w, "fused", "f32", "bf16", "xbc", False)
    t = fw.t
    H, P = w.nheads, w.headdim
    gs = H * P // w.ngroups
    wt = torch.ones(H * P, device=t["x"].device)
    # the fused workspace plus the per-(token, 64-channel block) sums of squares
    ws_n = torch.empty(fw.prob.workspace_size("fused") + 4 * w.tokens * (H * P // 64) + 256,
                       dtype=torch.uint8, device=t["x"].device)
    y = torch.empty_like(fw.out)

    def fused():
        ssd.ssd_forward_gated_norm(t["x"], t["B"], t["C"], t["dt"], t["A"], wt, gs, t["bias"],
                                   t["D"], t["z"], None, t["cu"], out=fw.out,
                                   final_states=fw.fin, workspace=ws_n)

    def two_calls():
        ssd.ssd_forward(t["x"], t["B"], t["C"], t["dt"], t["A"], t["bias"], t["D"], None, None,
                        t["cu"], w.chunk_size, out=y, final_states=fw.fin, algo="fused",
                        workspace=fw.ws)
        ssd.ssd_gated_rmsnorm_fwd(y, t["z"], wt, gs, out=fw.out)

    def timed(fn, n, cold):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            if cold:
                flush.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return round(float(np.median(ts)), 5)

    n = max(10, args.steps // 5)
    res = {"group_size": gs,
           "fused_cold_ms": timed(fused, n, True), "fused_warm_ms": timed(fused, n, False),
           "two_calls_cold_ms": timed(two_calls, n, True),
           "two_calls_warm_ms": timed(two_calls, n, False),
           "bytes_not_moved": 2 * 2 * w.tokens * H * P,
           "note": "fused: ssd_forward_gated_norm; two calls: ssd_forward (no gate) then "
                   "ssd_gated_rmsnorm_fwd (y and z read again); medians of event-timed calls"}
    del fw
    return res


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
    """HIP-event time of the backward (all gradients) on the same inputs, with
    an upstream gradient drawn from N(0, 1): ssd_backward_ex with AUTO (the
    per-chunk path where it applies) as the headline, the staged backward
    beside it; the forward+backward rate adds the forward step time measured
    above."""
    import torch
    g = torch.Generator(device=x.device).manual_seed(4)
    dout = torch.randn(x.shape, generator=g, device=x.device, dtype=torch.float32)
    prob = ssd.problem_from(x, B, w.chunk_size, cu_seqlens=cu, input_dt=args.input_dt)
    fused = x.dtype == torch.bfloat16 and w.headdim == 64 and w.dstate <= 128

    def timed(algo):
        ws = torch.empty(max(prob.backward_workspace_size(algo, x.dtype), 1), dtype=torch.uint8,
                         device=x.device)

        def bwd():
            return ssd.ssd_backward(x, B, C, dt, A, dout, dt_bias=bias, D=D, z=z, cu_seqlens=cu,
                                    chunk_size=w.chunk_size, workspace=ws,
                                    input_dt=args.input_dt, algo=algo)

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
        n = ws.numel()
        del ws
        return float(np.median(times)), n, len(times)

    bms, wsb, nst = timed("auto")
    sms, swsb, _ = timed("staged") if fused else (bms, wsb, nst)
    # the backward's algorithmic bytes: read x, B, C, dt, z (input dtype) and dout
    # (fp32); write dx, dB, dC, ddt, dz (fp32); per-head vectors are negligible
    tok = w.batch * w.seqlen
    H, P, G, N = w.nheads, w.headdim, w.ngroups, w.dstate
    e = 2 if w.dtype == "bf16" else 4
    zb = tok * H * P if w.has_z else 0
    alg = (e * (tok * H * P + 2 * tok * G * N + tok * H + zb) + 4 * tok * H * P
           + 4 * (tok * H * P + 2 * tok * G * N + tok * H + zb))
    return {"algo": "fused (per-chunk)" if fused else "staged",
            "bwd_ms": round(bms, 5), "fwd_ms": round(fwd_ms, 5),
            "bwd_algorithmic_bytes": alg,
            "bwd_hbm_frac": round(alg / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "fwd_bwd_ms": round(bms + fwd_ms, 5),
            "tokens_per_s": round(w.tokens / ((bms + fwd_ms) * 1e-3), 1),
            "workspace_MB": round(wsb / 1e6, 1),
            "staged_bwd_ms": round(sms, 5), "staged_workspace_MB": round(swsb / 1e6, 1),
            "steps": nst,
            "note": "median of event-timed backward calls (gradients allocated by the "
                    "binding inside the events), plus the timed forward step"}


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
