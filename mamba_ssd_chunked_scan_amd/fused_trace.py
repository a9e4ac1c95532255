"""Phase timeline of the fused forward (profiling build only).

    python -m mamba_ssd_chunked_scan_amd.fused_trace --build        # here: builds libssd_trace.so
    python -m mamba_ssd_chunked_scan_amd.fused_trace [--workload W] # on the GPU: runs and reports

The profiling library is libssd with -DSSD_FUSED_TRACE: every (unit, range)
item stores the device's 100 MHz clock (s_memrealtime) at the start and end of
its range aggregate (first launch) and inside that launch's first four chunk
steps, and at the start of the output launch, after its carry-in is loaded,
after each chunk and at its end, in a region at the end of its workspace.  The report gives, over the items of the last of
several forwards, the mean and spread of each phase and each launch's span.
"""
from __future__ import annotations

import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TRACE_LIB = os.path.join(HERE, "libssd_trace.so")
SLOTS = 64          # kFusedTraceSlots
TICK_NS = 10.0      # s_memrealtime runs at 100 MHz


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true")
    ap.add_argument("--workload", default="nemotron")
    ap.add_argument("--seqlen", type=int, default=0)
    ap.add_argument("--runs", type=int, default=5)
    args = ap.parse_args(argv)
    if args.build:
        from mamba_ssd_chunked_scan_amd import build
        print(build.build(variant="trace"))
        return 0

    import numpy as np
    import torch

    from mamba_ssd_chunked_scan_amd import ssd
    from mamba_ssd_chunked_scan_amd.inputs import WORKLOADS, make_inputs

    if not os.path.exists(TRACE_LIB):
        raise SystemExit(f"{TRACE_LIB} is not built (run with --build first)")
    ssd.LIB_PATH = TRACE_LIB
    w = WORKLOADS[args.workload]
    if args.seqlen:
        import dataclasses
        w = dataclasses.replace(w, seqlen=args.seqlen)
    inp = make_inputs(w)
    dev = "cuda"
    bf = torch.bfloat16
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, bf)
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev, torch.float32)
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    x, B, C, dt, z = t(inp.x), t(inp.B), t(inp.C), t(inp.dt), t(inp.z)
    prob = ssd.problem_from(x, B, 128, cu_seqlens=cu)
    need = prob.workspace_size("fused")
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for _ in range(args.runs):
        ssd.ssd_forward(x, B, C, dt, f(inp.A), f(inp.dt_bias), f(inp.D), z, cu_seqlens=cu,
                        chunk_size=128, algo="fused", workspace=ws)
    torch.cuda.synchronize()
    # the trace region is the workspace's last items * SLOTS words
    H, P = w.nheads, w.headdim
    U = H * ((P + 63) // 64)
    K = prob.num_chunks() if False else None  # (the plan is recomputed below)
    nc = -(-w.seqlen // 128)
    Kf = nc + w.nseq if (cu is not None) else w.batch * nc
    nr = max(1, min(512 // U, Kf))
    R = -(-Kf // nr)
    nr = -(-Kf // R)
    items = nr * U
    nbytes = items * SLOTS * 8
    region = ws[need - ((nbytes + 255) // 256) * 256:][:nbytes]
    tr = region.cpu().numpy().view(np.uint64).reshape(items, SLOTS).astype(np.float64)
    us = lambda v: v * TICK_NS / 1000.0
    has_agg = tr[:, 1] > 0
    t0 = tr[has_agg, 0].min() if has_agg.any() else tr[:, 2].min()
    rel = lambda v: us(v - t0)
    print(f"workload {w.name} T={w.seqlen}: {items} items = {U} units x {nr} ranges of {R} chunks")
    if has_agg.any():
        a0, a1 = tr[has_agg, 0], tr[has_agg, 1]
        print(f"aggregate launch: {has_agg.sum()} items, span {rel(a1.max()):.1f} us; "
              f"item mean {us((a1 - a0).mean()):.1f} max {us((a1 - a0).max()):.1f} us "
              f"({us((a1 - a0).mean()) / R:.2f} us per chunk)")
        # the aggregate launch's chunk steps (first four): barrier, staging,
        # load issue, barrier, decay weights, products
        names = ["barrier", "stage x/B", "issue loads", "barrier", "weights", "products"]
        ta = tr[has_agg]
        for k in range(4):
            prev = ta[:, 0] if k == 0 else ta[:, 32 + 6 * (k - 1) + 5]
            parts = []
            for m in range(6):
                cur = ta[:, 32 + 6 * k + m]
                parts.append(us(cur - prev).mean())
                prev = cur
            print(f"  step {k}: " + "  ".join(f"{n} {v:.2f}" for n, v in zip(names, parts))
                  + f"  (total {sum(parts):.2f} us)")
    s2, s3, se = tr[:, 2], tr[:, 3], tr[:, SLOTS - 2]
    print(f"output launch: starts {rel(s2.min()):.1f} .. {rel(s2.max()):.1f} us, "
          f"ends {rel(se.min()):.1f} .. {rel(se.max()):.1f} us (span {us(se.max() - s2.min()):.1f})")
    print(f"  carry-in        mean {us((s3 - s2).mean()):.2f}  max {us((s3 - s2).max()):.2f} us")
    ph = {n: [] for n in "ABCDE"}
    ck, k0 = [], []
    for i in range(items):
        r_ = i // U
        nch = min(R, Kf - r_ * R)
        prev = tr[i, 3]
        for k in range(min(nch, 10)):
            if k < 4:
                for m, n in enumerate("ABCDE"):
                    ph[n].append(us(tr[i, 4 + 5 * k + m] - prev))
                    prev = tr[i, 4 + 5 * k + m]
                d = sum(ph[n][-1] for n in "ABCDE")
            else:
                d = us(tr[i, 20 + k] - prev)
                prev = tr[i, 20 + k]
            ck.append(d)
            if k == 0:
                k0.append(d)
    ck = np.array(ck)
    print(f"  chunk           mean {ck.mean():.2f}  median {np.median(ck):.2f}  "
          f"first chunk mean {np.mean(k0):.2f} us")
    print("  phases (chunks 0-3): " + "  ".join(f"{n} {np.mean(ph[n]):.2f}" for n in "ABCDE")
          + " us  (A carry-in to LDS, B Y_off, C x/B to LDS, D state + C.B^T + Y_diag,"
          " E gate + store)")
    print(f"  item total      mean {us((se - s2).mean()):.1f}  max {us((se - s2).max()):.1f} us")
    # per range
    rix = np.arange(items) // U
    for r_ in range(nr):
        m = rix == r_
        print(f"  range {r_}: carry-in {us((s3[m] - s2[m]).mean()):5.2f}  item {us((se[m] - s2[m]).mean()):6.1f}"
              f"  ends mean {rel(se[m]).mean():6.1f} max {rel(se[m]).max():6.1f} us")
    return 0


if __name__ == "__main__":
    sys.exit(main())
