"""The single-pass forward (SSD_ALGO_FUSED) against the fp64 oracle, on the
shapes and sequence structures its work split depends on: partial 64-row P
slabs, every d_state tile width, long look-back chains, ranges of several
chunks, packed batches whose sequences start and end inside ranges (and empty
sequences and empty ranges), a workspace that starts out as garbage, and HIP
graph capture (both paths).
"""
import numpy as np
import pytest
import torch

from mamba_ssd_chunked_scan_amd import ssd
from helpers import (TOL_BF16_DESIGN, bf16_out_ok, device_inputs, err, make_inputs,
                     oracle_run, small_workload, to_np, with_initial_states)

pytestmark = pytest.mark.gpu


def run(inp, w, out_dtype=torch.float32, workspace=None, chunk_size=None, dt_dtype=None):
    dev = device_inputs(inp, torch.bfloat16)
    dt = dev["dt"] if dt_dtype is None else dev["dt"].to(dt_dtype)
    out, fin = ssd.ssd_forward(dev["x"], dev["B"], dev["C"], dt, dev["A"], dev["dt_bias"],
                               dev["D"], dev["z"], dev["initial_states"],
                               cu_seqlens=dev["cu_seqlens"],
                               chunk_size=chunk_size or w.chunk_size, out_dtype=out_dtype,
                               algo="fused", workspace=workspace)
    torch.cuda.synchronize()
    return out, fin


def check(y, f, ref, out_dtype=torch.float32):
    gy = to_np(y)
    if out_dtype == torch.float32:
        e = err(gy, ref.y)
        assert e <= TOL_BF16_DESIGN, f"output err {e:.3e}"
    else:
        okay, excess = bf16_out_ok(gy, ref.y, TOL_BF16_DESIGN)
        assert okay, f"bf16 output exceeds its bound by {excess:.3e}"
    ef = err(to_np(f), ref.final_states)
    assert ef <= TOL_BF16_DESIGN, f"final state err {ef:.3e}"


# (headdim, dstate): one and several P slabs, partial slabs, and the 32-, 64-
# and 128-wide d_state variants with unused tiles
SHAPES = [(16, 16), (48, 48), (64, 32), (80, 64), (128, 96), (256, 128), (64, 128), (32, 112)]


@pytest.mark.parametrize("P,N", SHAPES)
def test_shapes(P, N):
    w = small_workload(f"p{P}n{N}", seqlen=300, nheads=3, headdim=P, ngroups=1, dstate=N,
                       chunk_size=64)
    inp = with_initial_states(make_inputs(w))
    ref = oracle_run(inp)
    y, f = run(inp, w)
    check(y, f, ref)


def test_deep_lookback():
    # one unit: every 128-token chunk is its own range, so the last range sums
    # the aggregates of 39 predecessors
    w = small_workload("deep", seqlen=40 * 128 - 5, nheads=1, headdim=64, ngroups=1, dstate=64,
                       chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    ref = oracle_run(inp)
    y, f = run(inp, w)
    check(y, f, ref)


def test_multi_chunk_ranges():
    # 128 units: 16 chunks in 4 ranges of 4
    w = small_workload("ranges", seqlen=2048 - 37, nheads=128, headdim=64, ngroups=4, dstate=32,
                       chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    ref = oracle_run(inp)
    y, f = run(inp, w)
    check(y, f, ref)


# The plan aims at 512 (unit, range) workgroups: 512 units give one range (no
# aggregate launch), 256 give two (the second range takes the first one's
# aggregate as it stands, no carry launch) and 160 give three (the carry launch
# runs).  Six 128-token chunks; packed sequences start and end inside ranges.
FEW_RANGES = [(512, None), (256, None), (160, None), (512, (100, 200, 90, 300)),
              (256, (100, 200, 90, 300)), (160, (100, 200, 90, 300)), (160, (700, 0, 10))]


@pytest.mark.parametrize("H,seqlens", FEW_RANGES)
def test_one_two_three_ranges(H, seqlens):
    w = small_workload(f"r{H}", seqlen=690 if seqlens is None else sum(seqlens), nheads=H,
                       headdim=16, ngroups=4, dstate=16, chunk_size=128, seqlens=seqlens)
    inp = with_initial_states(make_inputs(w))
    ref = oracle_run(inp)
    y, f = run(inp, w)
    check(y, f, ref)


VARLEN = (300, 0, 1, 127, 128, 129, 1000, 0, 1315)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_packed_sequences_across_ranges(out_dtype):
    # 64 units, 27 real chunks in ranges of 5: sequences start and end inside
    # ranges, two are empty, and the last range slot has no chunk at all
    w = small_workload("varlen", seqlen=sum(VARLEN), nheads=64, headdim=16, ngroups=4,
                       dstate=16, chunk_size=64, seqlens=VARLEN)
    inp = with_initial_states(make_inputs(w))
    ref = oracle_run(inp)
    y, f = run(inp, w, out_dtype=out_dtype)
    check(y, f, ref, out_dtype)
    cu = inp.cu_seqlens
    for i in range(len(cu) - 1):
        if cu[i + 1] == cu[i]:
            assert np.array_equal(to_np(f[i]), inp.initial_states[i].astype(np.float64))


def test_garbage_workspace_and_reuse():
    w = small_workload("ws", seqlen=1000, nheads=16, headdim=64, ngroups=8, dstate=128,
                       chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    ref = oracle_run(inp)
    dev = device_inputs(inp, torch.bfloat16)
    prob = ssd.problem_from(dev["x"], dev["B"], 128)
    ws = torch.full((prob.workspace_size("fused"),), 0xFF, dtype=torch.uint8, device="cuda")
    y1, f1 = run(inp, w, workspace=ws)
    check(y1, f1, ref)
    y2, f2 = run(inp, w, workspace=ws)  # the workspace as the first call left it
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_chunk_size_is_internal():
    # the fused pass always works on 128-token chunks: the problem's chunk_size
    # changes nothing
    w = small_workload("cs", seqlen=777, nheads=8, headdim=32, ngroups=2, dstate=64,
                       chunk_size=64)
    inp = with_initial_states(make_inputs(w))
    ya, fa = run(inp, w, chunk_size=32)
    yb, fb = run(inp, w, chunk_size=256)
    assert torch.equal(ya, yb) and torch.equal(fa, fb)


def test_fp32_dt_with_bf16_inputs():
    # dt may come in fp32; the same values in bf16 give the same result
    w = small_workload("dt32", seqlen=500, nheads=4, headdim=64, ngroups=2, dstate=64,
                       chunk_size=128)
    inp = make_inputs(w)
    ya, fa = run(inp, w)
    yb, fb = run(inp, w, dt_dtype=torch.float32)
    assert torch.equal(ya, yb) and torch.equal(fa, fb)


def test_rejects_large_dstate():
    w = small_workload("n256", seqlen=64, nheads=1, headdim=16, ngroups=1, dstate=144,
                       chunk_size=64)
    inp = make_inputs(w)
    with pytest.raises(ssd.SSDError) as e:
        run(inp, w)
    assert e.value.status == 5


@pytest.mark.parametrize("algo", ["staged", "fused"])
def test_graph_capture_replays_match_eager(algo):
    # every ssd_* call is stream-ordered device work with no host
    # synchronisation or allocation, so a whole forward can be captured in a
    # HIP graph; each replay (with eager work in between) must reproduce the
    # eager result exactly
    w = small_workload("graph", seqlen=700, nheads=8, headdim=64, ngroups=2, dstate=64,
                       chunk_size=128, seqlens=(300, 0, 1, 399))
    inp = with_initial_states(make_inputs(w))
    dev = device_inputs(inp, torch.bfloat16)
    prob = ssd.problem_from(dev["x"], dev["B"], 128, cu_seqlens=dev["cu_seqlens"])
    ws = torch.empty(prob.workspace_size(algo), dtype=torch.uint8, device="cuda")
    out = torch.empty(dev["x"].shape, dtype=torch.float32, device="cuda")
    fin = torch.empty(dev["initial_states"].shape, dtype=torch.float32, device="cuda")

    def fwd():
        ssd.ssd_forward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"], dev["dt_bias"],
                        dev["D"], dev["z"], dev["initial_states"], cu_seqlens=dev["cu_seqlens"],
                        chunk_size=128, out=out, final_states=fin, algo=algo, workspace=ws)

    fwd()
    torch.cuda.synchronize()
    ref_out, ref_fin = out.clone(), fin.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    for _ in range(4):
        out.fill_(float("nan"))
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin)
        fwd()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
