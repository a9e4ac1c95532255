"""Streams, graphs and repeat runs of ssd_forward.

* Two forwards (fused and staged, each with its own workspace) on two streams
  at once give the bits of the same calls run one after the other
  (cudnn-frontend PR 1133, review "Validation": stream concurrency).
* A captured forward replays correctly when its input buffers are refilled
  between replays, and two graphs of the same call on different buffers
  interleave (pointer rebinding, graph replay).
* Repeated full-size fused calls are bit-identical to the first.
"""
import numpy as np
import pytest
import torch

from mamba_ssd_chunked_scan_amd import ssd
from mamba_ssd_chunked_scan_amd.inputs import WORKLOADS
from helpers import device_inputs, make_inputs, small_workload, with_initial_states

pytestmark = pytest.mark.gpu


def fwd(dev, algo, chunk_size=128, **kw):
    return ssd.ssd_forward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"], dev["dt_bias"],
                           dev["D"], dev["z"], dev["initial_states"],
                           cu_seqlens=dev["cu_seqlens"], chunk_size=chunk_size, algo=algo,
                           **kw)


# ------------------------------------------------------------------ streams

def test_two_streams_at_once_match_serial_runs():
    wa = small_workload("sa", seqlen=3000, nheads=32, headdim=64, ngroups=4, dstate=128,
                        chunk_size=128)
    wb = small_workload("sb", seqlen=2500, nheads=16, headdim=64, ngroups=2, dstate=64,
                        chunk_size=64, seqlens=(900, 1, 0, 1599), seed=9)
    da = device_inputs(with_initial_states(make_inputs(wa)), torch.bfloat16)
    db = device_inputs(with_initial_states(make_inputs(wb)), torch.bfloat16)
    ra = fwd(da, "fused")
    rb = fwd(db, "staged", chunk_size=64)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(5):
        with torch.cuda.stream(s1):
            oa = fwd(da, "fused", stream=s1)
        with torch.cuda.stream(s2):
            ob = fwd(db, "staged", chunk_size=64, stream=s2)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa[0], ra[0]) and torch.equal(oa[1], ra[1])
        assert torch.equal(ob[0], rb[0]) and torch.equal(ob[1], rb[1])


def test_backward_paths_on_two_streams_match_serial_runs():
    # the per-chunk and the staged backward at once on two streams (each call
    # allocates its own workspace and gradients on its stream), against the
    # same calls run one after the other
    w = small_workload("bs", seqlen=1500, nheads=16, headdim=64, ngroups=2, dstate=128,
                       chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    dev = device_inputs(inp, torch.bfloat16)
    g = torch.Generator(device="cuda").manual_seed(3)
    dout = torch.randn(dev["x"].shape, generator=g, device="cuda")

    def bwd(algo, stream=None):
        return ssd.ssd_backward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"], dout,
                                dt_bias=dev["dt_bias"], D=dev["D"], z=dev["z"],
                                initial_states=dev["initial_states"], chunk_size=128,
                                algo=algo, stream=stream)

    rf, rs = bwd("fused"), bwd("staged")
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            of = bwd("fused", stream=s1)
        with torch.cuda.stream(s2):
            os_ = bwd("staged", stream=s2)
        outs.append((of, os_))
    torch.cuda.synchronize()
    names = ("dx", "dB", "dC", "ddt", "dA", "ddt_bias", "dD", "dz", "dinitial_states")
    for of, os_ in outs:
        for n in names:
            assert torch.equal(getattr(of, n), getattr(rf, n)), n
            assert torch.equal(getattr(os_, n), getattr(rs, n)), n


def test_side_stream_temporaries_are_not_reused_early():
    # the binding allocates the workspace and outputs on the stream it launches
    # on; a busy current stream allocating and freeing at the same time must
    # not disturb a forward in flight on a side stream
    w = small_workload("side", seqlen=4096, nheads=32, headdim=64, ngroups=4, dstate=128,
                       chunk_size=128)
    dev = device_inputs(with_initial_states(make_inputs(w)), torch.bfloat16)
    ref = fwd(dev, "fused")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    results = []
    for _ in range(6):
        with torch.cuda.stream(s):
            results.append(fwd(dev, "fused", stream=s))
        junk = torch.empty(1 << 22, dtype=torch.uint8, device="cuda").fill_(0xFF)
        del junk
    torch.cuda.synchronize()
    for y, f in results:
        assert torch.equal(y, ref[0]) and torch.equal(f, ref[1])


# ------------------------------------------------------------------ graphs

@pytest.mark.parametrize("algo", ["staged", "fused"])
def test_graph_replays_with_refilled_and_rebound_buffers(algo):
    w = small_workload("rebind", seqlen=900, nheads=8, headdim=64, ngroups=2, dstate=64,
                       chunk_size=128, seqlens=(400, 0, 3, 497))
    sets = [device_inputs(with_initial_states(make_inputs(w, seed=s), seed=s), torch.bfloat16)
            for s in (1, 2, 3)]
    prob = ssd.problem_from(sets[0]["x"], sets[0]["B"], 128, cu_seqlens=sets[0]["cu_seqlens"])
    ws = torch.empty(prob.workspace_size(algo), dtype=torch.uint8, device="cuda")
    bufs = [(torch.empty(d["x"].shape, dtype=torch.float32, device="cuda"),
             torch.empty(d["initial_states"].shape, dtype=torch.float32, device="cuda"))
            for d in sets[:2]]

    def call(d, ob):
        fwd(d, algo, out=ob[0], final_states=ob[1], workspace=ws)

    eager = []
    for d in sets:
        o, f = fwd(d, algo, out_dtype=torch.float32)
        eager.append((o.clone(), f.clone()))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(sets[0], bufs[0])
        call(sets[1], bufs[1])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for k in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(sets[k], bufs[k])
        graphs.append(g)
    # the two graphs (one workspace, different input and output buffers)
    # interleaved, with eager work in between
    for k in (0, 1, 1, 0):
        for t in bufs[k]:
            t.fill_(float("nan"))
        graphs[k].replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[k][0], eager[k][0]) and torch.equal(bufs[k][1], eager[k][1])
        fwd(sets[2], algo, out_dtype=torch.float32)
    # graph 0's inputs refilled in place with the third input set
    for name in ("x", "B", "C", "dt", "z", "A", "dt_bias", "D", "initial_states"):
        sets[0][name].copy_(sets[2][name])
    graphs[0].replay()
    torch.cuda.synchronize()
    assert torch.equal(bufs[0][0], eager[2][0]) and torch.equal(bufs[0][1], eager[2][1])


# ------------------------------------------------------------------ bounded repeat

@pytest.mark.parametrize("shape", ["nemotron", "deep_lookback"])
def test_repeated_fused_calls_are_bit_identical(shape):
    if shape == "nemotron":
        w = WORKLOADS["nemotron"]
        inp = make_inputs(w)
    else:
        w = small_workload("deep", seqlen=200 * 128 - 9, nheads=1, headdim=64, ngroups=1,
                           dstate=128, chunk_size=128)
        inp = with_initial_states(make_inputs(w))
    dev = device_inputs(inp, torch.bfloat16, packed_xbc=True)
    prob = ssd.problem_from(dev["x"], dev["B"], 128, cu_seqlens=dev["cu_seqlens"])
    ws = torch.empty(prob.workspace_size("fused"), dtype=torch.uint8, device="cuda")
    first, first_f = fwd(dev, "fused", workspace=ws)
    out = torch.empty_like(first)
    fin = torch.empty_like(first_f)
    for i in range(200):
        fwd(dev, "fused", out=out, final_states=fin, workspace=ws)
        same = torch.equal(out, first) and torch.equal(fin, first_f)
        assert same, f"call {i} differs from the first"
