"""ssd_backward on the GPU against the fp64 backward oracle (oracle.ssd_bwd).

Every gradient (dx, dB, dC, ddt, dA, ddt_bias, dD, dz, dinitial_states) is
compared with err() = max |gpu - ref| / RMS(ref) over the whole tensor.  The
backward runs in fp32 after the inputs (fp32 chunk states and matrix
products), so every gradient of an fp32 problem is held to the fp32 gate
(1e-4) and every gradient of a bf16 problem to the forward's bf16 design bound
(2e-3).
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_chunked_scan_amd import ssd
from mamba_ssd_chunked_scan_amd.inputs import WORKLOADS
from helpers import (TOL_BF16_DESIGN, TOL_F32, device_inputs, err, head_slice, in_dtype,
                     make_inputs, small_workload, to_dev, to_np, with_initial_states)

pytestmark = pytest.mark.gpu

NAMES = ("dx", "dB", "dC", "ddt", "dA", "ddt_bias", "dD", "dz", "dinitial_states")


def upstream(inp, seed=123, dfinal=True):
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal(inp.x.shape)
    nseq = (len(inp.cu_seqlens) - 1) if inp.cu_seqlens is not None else inp.x.shape[0]
    H, P = inp.x.shape[-2:]
    N = inp.B.shape[-1]
    dfin = rng.standard_normal((nseq, H, P, N)) if dfinal else None
    return dout, dfin


def run_both(w, inp, dout, dfin, dt_limit=None, dt_softplus=True):
    ref = oracle.ssd_bwd(inp.x, inp.B, inp.C, inp.dt, inp.A, dout, dt_bias=inp.dt_bias, D=inp.D,
                         z=inp.z, initial_states=inp.initial_states, dfinal_states=dfin,
                         cu_seqlens=inp.cu_seqlens, dt_softplus=dt_softplus, dt_limit=dt_limit)
    dtype = in_dtype(w)
    dev = device_inputs(inp, dtype)
    g = ssd.ssd_backward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"],
                         to_dev(dout, torch.float32), dt_bias=dev["dt_bias"], D=dev["D"],
                         z=dev["z"], initial_states=dev["initial_states"],
                         dfinal_states=to_dev(dfin, torch.float32),
                         cu_seqlens=dev["cu_seqlens"], chunk_size=w.chunk_size,
                         dt_softplus=dt_softplus, dt_limit=dt_limit)
    torch.cuda.synchronize()
    return g, ref


def check(g, ref, tol):
    errs = {}
    for n in NAMES:
        a, r = getattr(g, n), getattr(ref, n)
        if r is None:
            assert a is None, n
            continue
        errs[n] = err(to_np(a), r)
    print({n: f"{e:.2e}" for n, e in errs.items()})
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"gradients over {tol:g}: {bad} (all: {errs})"


@pytest.mark.parametrize("dtype,tol", [("f32", TOL_F32), ("bf16", TOL_BF16_DESIGN)])
def test_batch_all_options(dtype, tol):
    w = small_workload("bwd", batch=2, seqlen=300, nheads=4, headdim=32, ngroups=2, dstate=32,
                       chunk_size=64, dtype=dtype)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    check(*run_both(w, inp, dout, dfin), tol)


VARLEN = (300, 0, 1, 127, 128, 129, 0, 500)


def test_packed_sequences():
    w = small_workload("bwd_varlen", seqlen=sum(VARLEN), nheads=4, headdim=16, ngroups=2,
                       dstate=16, chunk_size=64, dtype="f32", seqlens=VARLEN)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    g, ref = run_both(w, inp, dout, dfin)
    check(g, ref, TOL_F32)
    # an empty sequence passes its final-state gradient straight through
    cu = inp.cu_seqlens
    for i in range(len(cu) - 1):
        if cu[i + 1] == cu[i]:
            assert np.array_equal(to_np(g.dinitial_states[i]), dfin[i].astype(np.float32))


def test_no_gate_no_skip_no_states():
    w = small_workload("bwd_plain", seqlen=257, nheads=2, headdim=16, ngroups=1, dstate=48,
                       chunk_size=32, dtype="f32", has_D=False, has_z=False)
    inp = make_inputs(w)
    dout, _ = upstream(inp, dfinal=False)
    check(*run_both(w, inp, dout, None), TOL_F32)


def test_clamp_and_shapes():
    # odd heads per group, P != N, clamp active on part of the tokens
    w = small_workload("bwd_clamp", seqlen=200, nheads=6, headdim=48, ngroups=2, dstate=64,
                       chunk_size=128, dtype="f32")
    inp = with_initial_states(make_inputs(w))
    delta = oracle.step_size(inp.dt, inp.dt_bias)
    lim = tuple(float(v) for v in np.quantile(delta, [0.2, 0.8]))
    dout, dfin = upstream(inp)
    g, ref = run_both(w, inp, dout, dfin, dt_limit=lim)
    check(g, ref, TOL_F32)
    clamped = (delta < lim[0]) | (delta > lim[1])
    assert np.all(to_np(g.ddt)[clamped] == 0.0)


def test_without_softplus():
    w = small_workload("bwd_nosp", seqlen=150, nheads=2, headdim=16, ngroups=2, dstate=16,
                       chunk_size=64, dtype="f32")
    inp = with_initial_states(make_inputs(w))
    inp.dt = (np.abs(inp.dt) * 0.05 + 0.01).astype(inp.dt.dtype)
    inp.dt_bias = np.zeros_like(inp.dt_bias)
    dout, dfin = upstream(inp)
    check(*run_both(w, inp, dout, dfin, dt_softplus=False), TOL_F32)


def test_bit_identical_repeats():
    w = small_workload("bwd_rep", seqlen=400, nheads=4, headdim=32, ngroups=2, dstate=32,
                       chunk_size=64, dtype="bf16")
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    dev = device_inputs(inp, torch.bfloat16)
    args = (dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"], to_dev(dout, torch.float32))
    kw = dict(dt_bias=dev["dt_bias"], D=dev["D"], z=dev["z"],
              initial_states=dev["initial_states"], dfinal_states=to_dev(dfin, torch.float32),
              chunk_size=64)
    g1 = ssd.ssd_backward(*args, **kw)
    g2 = ssd.ssd_backward(*args, **kw)
    torch.cuda.synchronize()
    for n in NAMES:
        a, b = getattr(g1, n), getattr(g2, n)
        assert torch.equal(a, b), n


def test_nemotron_dims_sampled_group():
    # full Nemotron-Nano dims (8192 tokens, 64 heads x 64, d_state 128, 8
    # groups, chunk 128, bf16); the oracle runs on one group's 8 heads, which
    # fixes that group's dB and dC and every per-head gradient of its heads
    w = WORKLOADS["nemotron"]
    inp = make_inputs(w)
    dout, dfin = upstream(inp, seed=7)
    dev = device_inputs(inp, torch.bfloat16)
    g = ssd.ssd_backward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"],
                         to_dev(dout, torch.float32), dt_bias=dev["dt_bias"], D=dev["D"],
                         z=dev["z"], dfinal_states=to_dev(dfin, torch.float32),
                         chunk_size=w.chunk_size)
    torch.cuda.synchronize()
    grp = 3
    hpg = w.nheads // w.ngroups
    heads = list(range(grp * hpg, (grp + 1) * hpg))
    sub = head_slice(inp, heads)
    ref = oracle.ssd_bwd(sub.x, sub.B[:, :, :1], sub.C[:, :, :1], sub.dt, sub.A, dout[:, :, heads],
                         dt_bias=sub.dt_bias, D=sub.D, z=sub.z, dfinal_states=dfin[:, heads],
                         threads=8)
    got = dict(dx=g.dx[:, :, heads], dB=g.dB[:, :, grp:grp + 1], dC=g.dC[:, :, grp:grp + 1],
               ddt=g.ddt[:, :, heads], dA=g.dA[heads], ddt_bias=g.ddt_bias[heads],
               dD=g.dD[heads], dz=g.dz[:, :, heads],
               dinitial_states=g.dinitial_states[:, heads])
    errs = {n: err(to_np(got[n]), getattr(ref, n)) for n in got}
    print({n: f"{e:.2e}" for n, e in errs.items()})
    bad = {n: e for n, e in errs.items() if not e <= TOL_BF16_DESIGN}
    assert not bad, f"{bad} (all: {errs})"


@pytest.mark.parametrize("case", ["strong_decay", "no_decay", "weak_positive"])
def test_decay_rates(case):
    # A = -1e4 (every step forgets the past: the step-size gradients nearly
    # vanish, which a form with cancelling terms would get wrong), A = 0 (a
    # pure prefix sum: the raw dt gets no gradient, A still does) and a weakly
    # growing state
    w = small_workload(f"bwd_{case}", seqlen=190, nheads=4, headdim=16, ngroups=2, dstate=32,
                       chunk_size=64, dtype="f32")
    inp = with_initial_states(make_inputs(w))
    inp.A = np.full_like(inp.A, {"strong_decay": -1e4, "no_decay": 0.0, "weak_positive": 0.01}[case])
    dout, dfin = upstream(inp)
    g, ref = run_both(w, inp, dout, dfin)
    if case == "no_decay":
        assert np.all(to_np(g.ddt) == 0.0) and np.all(to_np(g.ddt_bias) == 0.0)
        g.ddt, ref.ddt = None, None
        g.ddt_bias, ref.ddt_bias = None, None
    check(g, ref, TOL_F32)
