"""Parity of the complex-A forward (ssd_complex_forward) with the fp64 oracle.

The oracle is the sequential complex recurrence (SSD Reference, "Math" with
"_discretise"), pinned in test_oracle_complex_pins.py.  Inputs are complex64 /
float32, so the gate is the fp32 one: max|gpu - ref| / RMS(ref) <= 1e-4, for
the real output (the page's chunkwise return contract), the full complex
output and the final state.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL_F32, err
from mamba_ssd_chunked_scan_amd import ssd
from mamba_ssd_chunked_scan_amd.inputs import (COMPLEX_WORKLOADS, ComplexWorkload,
                                               make_complex_inputs)

pytestmark = pytest.mark.gpu


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run(inp, C, out_complex=False, use_h0=True, views=None):
    x, B, Cm = (dev(inp.x), dev(inp.B), dev(inp.C)) if views is None else views
    y, fin = ssd.ssd_complex_forward(x, B, Cm, dev(inp.dt), dev(inp.A),
                                     initial_states=dev(inp.h0) if use_h0 else None,
                                     chunk_size=C, out_complex=out_complex)
    torch.cuda.synchronize()
    return y.cpu().numpy(), fin.cpu().numpy()


def reference(inp, use_h0=True):
    return oracle.ssd_complex_fwd(inp.x, inp.B, inp.C, inp.dt, inp.A,
                                  initial_states=inp.h0 if use_h0 else None)


def check(y, fin, r, out_complex):
    ry = r.y if out_complex else r.y.real
    e_y = err(y.view(np.float32), ry.view(np.float64)) if out_complex else err(y, ry)
    e_f = err(fin.view(np.float32), r.final_states.view(np.float64))
    print(f"complex forward: out err {e_y:.2e}, final-state err {e_f:.2e}")
    assert e_y <= TOL_F32 and e_f <= TOL_F32, (e_y, e_f)


@pytest.mark.parametrize("C", [32, 64, 128, 256])
@pytest.mark.parametrize("out_complex", [False, True])
def test_small_every_chunk_size(C, out_complex):
    # several chunks, a ragged tail (300 = 4 x 64 + 44), an initial state
    inp = make_complex_inputs(COMPLEX_WORKLOADS["complex_tiny"])
    y, fin = run(inp, C, out_complex)
    check(y, fin, reference(inp), out_complex)


@pytest.mark.parametrize("shape", [
    (1, 1, 2, 16, 16, 64),     # a single token
    (1, 64, 2, 16, 16, 64),    # exactly one chunk
    (2, 65, 2, 48, 80, 32),    # one token past a chunk edge; uneven tile counts
    (1, 200, 5, 128, 128, 64), # the largest head and state dims
    (3, 129, 1, 16, 128, 128),
])
def test_shapes(shape):
    b, T, H, P, N, C = shape
    w = ComplexWorkload("shape", b, T, H, P, N, C, seed=T * 7 + P, initial_states=True)
    inp = make_complex_inputs(w)
    for oc in (False, True):
        y, fin = run(inp, C, oc)
        check(y, fin, reference(inp), oc)


def test_no_initial_state_and_no_tokens():
    w = ComplexWorkload("noh0", 2, 190, 3, 32, 48, 64, seed=5)
    inp = make_complex_inputs(w)
    y, fin = run(inp, 64, use_h0=False)
    check(y, fin, reference(inp, use_h0=False), False)
    # T = 0: the final state is the initial state
    w0 = ComplexWorkload("empty", 2, 0, 3, 16, 16, 64, seed=6, initial_states=True)
    inp0 = make_complex_inputs(w0)
    y0, fin0 = run(inp0, 64)
    assert y0.shape == (2, 0, 3, 16)
    assert np.array_equal(fin0, inp0.h0)


def test_strided_views_of_one_buffer():
    # x, B, C as views into one (b, T, H, P + 2N) complex buffer
    w = ComplexWorkload("views", 2, 250, 4, 32, 16, 64, seed=9, initial_states=True)
    inp = make_complex_inputs(w)
    P, N = w.headdim, w.dstate
    packed = np.concatenate([inp.x, inp.B, inp.C], axis=-1)
    t = dev(packed)
    views = (t[..., :P], t[..., P:P + N], t[..., P + N:])
    y, fin = run(inp, 64, views=views)
    check(y, fin, reference(inp), False)


def test_decay_extremes_and_pure_rotation():
    # very strong decay (memoryless), a pure rotation (Re A = 0: no decay at all)
    w = ComplexWorkload("ext", 1, 300, 4, 16, 16, 64, seed=13, initial_states=True)
    inp = make_complex_inputs(w)
    inp.A = np.array([-1e4 + 0.5j, 0.0 + 2.0j, -1e-3 - 3.0j, 0.01 + 0.0j], dtype=np.complex64)
    y, fin = run(inp, 64)
    check(y, fin, reference(inp), False)


def test_run_to_run_bit_identical():
    inp = make_complex_inputs(COMPLEX_WORKLOADS["complex_tiny"])
    a = run(inp, 64, True)
    b = run(inp, 64, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_434m_config_sampled():
    # the SSD Reference's 434M shape, on the GPU in full; the oracle on sampled
    # (batch row, head) pairs (heads and rows are independent)
    w = COMPLEX_WORKLOADS["complex_434m"]
    inp = make_complex_inputs(w)
    y, fin = run(inp, w.chunk_size, use_h0=False)
    rows, heads = [0, 5], [0, 9, 15]
    sub = lambda a: a[rows][:, :, heads]
    r = oracle.ssd_complex_fwd(sub(inp.x), sub(inp.B), sub(inp.C), sub(inp.dt), inp.A[heads])
    e_y = err(y[rows][:, :, heads], r.y.real)
    e_f = err(fin[rows][:, heads].view(np.float32), r.final_states.view(np.float64))
    print(f"434M sampled: out err {e_y:.2e}, final-state err {e_f:.2e}")
    assert e_y <= TOL_F32 and e_f <= TOL_F32


def test_stage_intermediates():
    # chunk states = the recurrence run on each chunk alone from zero; after the
    # pass, carry-in states = the recurrence's state at each chunk's start
    w = ComplexWorkload("stages", 2, 150, 2, 16, 32, 64, seed=21, initial_states=True)
    inp = make_complex_inputs(w)
    prob = ssd.ComplexProblem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk_size)
    nc = -(-w.seqlen // w.chunk_size)
    x, B, C, dt, A, h0 = (dev(inp.x), dev(inp.B), dev(inp.C), dev(inp.dt), dev(inp.A),
                          dev(inp.h0))
    st = torch.empty((w.batch * nc, w.nheads, w.headdim, w.dstate), dtype=torch.complex64,
                     device="cuda")
    lam = torch.empty((w.nheads, w.batch * nc), dtype=torch.float32, device="cuda")
    ssd.ssd_complex_chunk_state(prob, x, B, dt, A, st, lam)
    torch.cuda.synchronize()
    S = st.cpu().numpy().reshape(w.batch, nc, w.nheads, w.headdim, w.dstate)
    for c in range(nc):
        t0, t1 = c * 64, min(150, c * 64 + 64)
        sl = lambda a: a[:, t0:t1]
        r = oracle.ssd_complex_fwd(sl(inp.x), sl(inp.B), sl(inp.C), sl(inp.dt), inp.A)
        assert err(S[:, c].view(np.float32), r.final_states.view(np.float64)) <= TOL_F32
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.complex64,
                      device="cuda")
    ssd.ssd_complex_state_passing(prob, A, lam, st, h0, fin)
    torch.cuda.synchronize()
    Hin = st.cpu().numpy().reshape(w.batch, nc, w.nheads, w.headdim, w.dstate)
    assert np.array_equal(Hin[:, 0], inp.h0)
    for c in range(1, nc):
        sl = lambda a: a[:, :c * 64]
        r = oracle.ssd_complex_fwd(sl(inp.x), sl(inp.B), sl(inp.C), sl(inp.dt), inp.A,
                                   initial_states=inp.h0)
        assert err(Hin[:, c].view(np.float32), r.final_states.view(np.float64)) <= TOL_F32
    out = torch.empty((w.batch, w.seqlen, w.nheads, w.headdim), dtype=torch.complex64,
                      device="cuda")
    ssd.ssd_complex_chunk_scan(prob, x, B, C, dt, A, st, out)
    torch.cuda.synchronize()
    y, f2 = run(inp, 64, out_complex=True)
    assert np.array_equal(out.cpu().numpy(), y) and np.array_equal(fin.cpu().numpy(), f2)


def test_graph_capture_replays_match_eager():
    # the complex forward and the gated RMSNorm (forward and backward) are
    # stream-ordered device work with caller-owned buffers, so they can be
    # captured in a HIP graph; every replay, with eager work in between, must
    # reproduce the eager results exactly
    inp = make_complex_inputs(COMPLEX_WORKLOADS["complex_tiny"])
    x, B, C, dt, A, h0 = (dev(inp.x), dev(inp.B), dev(inp.C), dev(inp.dt), dev(inp.A),
                          dev(inp.h0))
    prob = ssd.ComplexProblem(*inp.x.shape[:1], inp.x.shape[1], inp.x.shape[2], inp.x.shape[3],
                              inp.B.shape[3], 64)
    ws = torch.empty(max(prob.workspace_size(), 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(inp.x.shape, dtype=torch.complex64, device="cuda")
    fin = torch.empty(inp.h0.shape, dtype=torch.complex64, device="cuda")
    rng = np.random.default_rng(3)
    ny, nz, ndo = (torch.from_numpy(rng.standard_normal((1, 80, 4, 64)).astype(np.float32)).cuda()
                   for _ in range(3))
    nw = torch.from_numpy((1.0 + 0.2 * rng.standard_normal(256)).astype(np.float32)).cuda()
    nout = torch.empty_like(ny)
    ndy, ndz, ndw = torch.empty_like(ny), torch.empty_like(ny), torch.empty_like(nw)
    nws = torch.empty(max(ssd.gated_rmsnorm_bwd_workspace_size(ny, 128), 1), dtype=torch.uint8,
                      device="cuda")

    def work():
        ssd.ssd_complex_forward(x, B, C, dt, A, initial_states=h0, chunk_size=64,
                                out_complex=True, out=out, final_states=fin, workspace=ws)
        ssd.ssd_gated_rmsnorm_fwd(ny, nz, nw, 128, out=nout)
        ssd.ssd_gated_rmsnorm_bwd(ny, nz, nw, ndo, 128, workspace=nws, dy=ndy, dz=ndz, dw=ndw)

    bufs = (out, fin, nout, ndy, ndz, ndw)
    work()
    torch.cuda.synchronize()
    refs = [t.clone() for t in bufs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for _ in range(4):
        for t in bufs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(bufs, refs):
            assert torch.equal(t, r)
        work()  # eager work between replays
        torch.cuda.synchronize()
        for t, r in zip(bufs, refs):
            assert torch.equal(t, r)


@pytest.mark.parametrize("C", [32, 64, 256])
def test_packed_sequences(C):
    # sequences packed on one token axis (cu_seqlens): an empty one, a single
    # token, exact multiples of the chunk and ragged tails; each starts from its
    # own initial state
    lens = [1, 0, C - 1, C, C + 1, 2 * C + 3, 37]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    w = ComplexWorkload("packed", 1, T, 3, 32, 16, C, seed=31 + C)
    inp = make_complex_inputs(w)
    x, B, Cm, dt = inp.x[0], inp.B[0], inp.C[0], inp.dt[0]
    rng = np.random.default_rng(C)
    h0 = (rng.standard_normal((len(lens), 3, 32, 16))
          + 1j * rng.standard_normal((len(lens), 3, 32, 16))).astype(np.complex64)
    cu_dev = torch.tensor(cu, dtype=torch.int32, device="cuda")
    y, fin = ssd.ssd_complex_forward(dev(x), dev(B), dev(Cm), dev(dt), dev(inp.A),
                                     initial_states=dev(h0), chunk_size=C, out_complex=True,
                                     cu_seqlens=cu_dev)
    torch.cuda.synchronize()
    y, fin = y.cpu().numpy(), fin.cpu().numpy()
    ref = oracle.ssd_complex_fwd(x, B, Cm, dt, inp.A, initial_states=h0, cu_seqlens=cu)
    check(y, fin, ref, True)
    # every sequence run on its own in batch mode gives the same bits
    for i, L in enumerate(lens):
        a, b_ = int(cu[i]), int(cu[i + 1])
        if L == 0:
            assert np.array_equal(fin[i], h0[i])
            continue
        yi, fi = ssd.ssd_complex_forward(dev(x[None, a:b_]), dev(B[None, a:b_]),
                                         dev(Cm[None, a:b_]), dev(dt[None, a:b_]), dev(inp.A),
                                         initial_states=dev(h0[i:i + 1]), chunk_size=C,
                                         out_complex=True)
        torch.cuda.synchronize()
        assert np.array_equal(yi.cpu().numpy()[0], y[a:b_])
        assert np.array_equal(fi.cpu().numpy()[0], fin[i])


def test_long_sequence_more_than_256_chunks():
    # 300 chunks in one sequence: the pass over chunks takes its decays in blocks of
    # 256, so the second block is exercised (and a packed batch around it)
    T = 64 * 300 - 17
    w = ComplexWorkload("long", 1, T, 2, 16, 16, 64, seed=77, initial_states=True)
    inp = make_complex_inputs(w)
    y, fin = run(inp, 64, out_complex=True)
    check(y, fin, reference(inp), True)
    lens = [5, T - 5 - 64, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x, B, Cm, dt = inp.x[0], inp.B[0], inp.C[0], inp.dt[0]
    h0 = np.repeat(inp.h0, 3, axis=0)
    yp, fp = ssd.ssd_complex_forward(dev(x), dev(B), dev(Cm), dev(dt), dev(inp.A),
                                     initial_states=dev(h0), chunk_size=64, out_complex=True,
                                     cu_seqlens=torch.tensor(cu, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    ref = oracle.ssd_complex_fwd(x, B, Cm, dt, inp.A, initial_states=h0, cu_seqlens=cu)
    check(yp.cpu().numpy(), fp.cpu().numpy(), ref, True)
