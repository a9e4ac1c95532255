"""The step size on the input term (problem.input_dt: S = exp(delta A) S +
delta x (outer) B, the skip on the raw x) against the fp64 oracle with the same
option, through the C ABI: the two stages it changes (chunk state, chunk scan)
on the oracle's intermediates, the staged and fused forward end to end, and
the backward.  The oracle's option is pinned in tests/test_oracle_pins.py and
tests/test_oracle_bwd_pins.py.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_chunked_scan_amd import ssd
from mamba_ssd_chunked_scan_amd.inputs import WORKLOADS
from helpers import (TOL_BF16_DESIGN, TOL_F32, bf16_out_ok, device_inputs, err, head_slice,
                     in_dtype, make_inputs, oracle_run, small_workload, to_dev, to_np,
                     with_initial_states)

pytestmark = pytest.mark.gpu

CASES = {
    "f32_ragged": small_workload("idt_f32", batch=2, seqlen=150, nheads=4, headdim=16,
                                 ngroups=2, dstate=32, chunk_size=64, dtype="f32"),
    "bf16_c128": small_workload("idt_bf16", seqlen=520, nheads=4, headdim=64, ngroups=1,
                                dstate=128, chunk_size=128),
    "bf16_c32": small_workload("idt_c32", seqlen=77, nheads=6, headdim=32, ngroups=3,
                               dstate=48, chunk_size=32),
    "packed": small_workload("idt_packed", seqlen=700, nheads=4, headdim=32, ngroups=2,
                             dstate=32, chunk_size=64, seqlens=(1, 63, 64, 65, 0, 200, 307)),
}


def tol_of(w):
    return TOL_F32 if w.dtype == "f32" else TOL_BF16_DESIGN


def setup(name):
    w = CASES[name]
    inp = with_initial_states(make_inputs(w))
    dev = device_inputs(inp, in_dtype(w))
    prob = ssd.problem_from(dev["x"], dev["B"], w.chunk_size, cu_seqlens=dev["cu_seqlens"],
                            input_dt=True)
    if inp.cu_seqlens is not None:
        prob.chunk_meta = ssd.ssd_varlen_chunk_meta(prob)
        meta = oracle.varlen_chunk_meta(inp.cu_seqlens, w.chunk_size)
        tok = lambda a: a
    else:
        meta = oracle.batch_chunk_meta(w.batch, w.seqlen, w.chunk_size)
        tok = lambda a: None if a is None else a.reshape((-1,) + a.shape[2:])
    return w, inp, dev, prob, meta, tok


def chunked(v, meta, K, C):
    """(ntok, H) per-token values -> (K, H, C), zero past each chunk's end."""
    out = np.zeros((K, v.shape[1], C))
    for j in range(meta.nchunks):
        s, L = meta.start[j], meta.length[j]
        out[j, :, :L] = v[s:s + L].T
    return out


def stage_inputs(w, inp, prob, meta, tok):
    K = prob.num_chunks()
    cs = np.zeros((K, w.nheads, w.chunk_size))
    cs[:meta.nchunks] = oracle.chunk_cumsum(tok(inp.dt), inp.A, meta, w.chunk_size,
                                            dt_bias=inp.dt_bias)
    delta = oracle.step_size(tok(inp.dt), inp.dt_bias)
    return (to_dev(cs, torch.float32), to_dev(chunked(delta, meta, K, w.chunk_size), torch.float32))


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_state(name):
    w, inp, dev, prob, meta, tok = setup(name)
    cs, dtc = stage_inputs(w, inp, prob, meta, tok)
    got = to_np(ssd.ssd_chunk_state(prob, dev["x"], dev["B"], cs, dt_chunk=dtc))[:meta.nchunks]
    torch.cuda.synchronize()
    ref = oracle.chunk_states(tok(inp.x), tok(inp.B), tok(inp.dt), inp.A, meta,
                              dt_bias=inp.dt_bias, input_dt=True)
    assert err(got, ref) <= tol_of(w)
    # without it the states differ by O(1): the option is really on
    plain = oracle.chunk_states(tok(inp.x), tok(inp.B), tok(inp.dt), inp.A, meta,
                                dt_bias=inp.dt_bias)
    assert err(got, plain) > 0.05


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_scan(name):
    w, inp, dev, prob, meta, tok = setup(name)
    cs, dtc = stage_inputs(w, inp, prob, meta, tok)
    r = oracle_run(inp, chunk_size=w.chunk_size, input_dt=True)
    K = prob.num_chunks()
    cb = torch.zeros((K, w.ngroups, w.chunk_size, w.chunk_size), dtype=torch.float32,
                     device="cuda")
    cb[:meta.nchunks] = to_dev(oracle.bmm_chunk(tok(inp.C), tok(inp.B), meta, w.chunk_size),
                               torch.float32)
    hin = torch.zeros((K, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")
    hin[:meta.nchunks] = to_dev(oracle.carry_in_states(r.chunk_end_states, meta,
                                                       inp.initial_states), torch.float32)
    out = ssd.ssd_chunk_scan(prob, cb, dev["x"], dev["C"], cs, hin, D=dev["D"], z=dev["z"],
                             out_dtype=torch.float32, dt_chunk=dtc)
    torch.cuda.synchronize()
    assert err(to_np(out), r.y) <= tol_of(w)


def test_stage_calls_need_dt_chunk():
    w, inp, dev, prob, meta, tok = setup("f32_ragged")
    cs, _ = stage_inputs(w, inp, prob, meta, tok)
    with pytest.raises(RuntimeError, match="dt_chunk"):
        ssd.ssd_chunk_state(prob, dev["x"], dev["B"], cs)


def run_fwd(w, inp, algo, out_dtype=torch.float32, **kw):
    dev = device_inputs(inp, in_dtype(w))
    out, fin = ssd.ssd_forward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"],
                               dev["dt_bias"], dev["D"], dev["z"], dev["initial_states"],
                               cu_seqlens=dev["cu_seqlens"], chunk_size=w.chunk_size,
                               out_dtype=out_dtype, algo=algo, input_dt=True, **kw)
    torch.cuda.synchronize()
    return to_np(out), to_np(fin)


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("algo", ["staged", "fused", "auto"])
def test_forward(name, algo):
    w = CASES[name]
    if algo == "fused" and w.dtype == "f32":
        algo = "auto"   # fused refuses fp32 inputs (tested in test_gpu_forward.py); auto routes
    inp = with_initial_states(make_inputs(w))
    ref = oracle_run(inp, input_dt=True)
    y, fin = run_fwd(w, inp, algo)
    assert err(y, ref.y) <= tol_of(w)
    assert err(fin, ref.final_states) <= tol_of(w)


@pytest.mark.parametrize("algo", ["staged", "fused"])
def test_forward_clamp_and_bf16_out(algo):
    w = CASES["bf16_c128"]
    inp = with_initial_states(make_inputs(w))
    delta = oracle.step_size(inp.dt, inp.dt_bias)
    lim = tuple(float(v) for v in np.quantile(delta, [0.2, 0.8]))
    ref = oracle_run(inp, dt_limit=lim, input_dt=True)
    y, fin = run_fwd(w, inp, algo, out_dtype=torch.bfloat16, dt_limit=lim)
    okay, excess = bf16_out_ok(y, ref.y, TOL_BF16_DESIGN)
    assert okay, excess
    assert err(fin, ref.final_states) <= TOL_BF16_DESIGN


def test_fused_rejects_possibly_negative_steps():
    w = CASES["bf16_c128"]
    inp = make_inputs(w)
    with pytest.raises(RuntimeError, match="delta >= 0"):
        run_fwd(w, inp, "fused", dt_softplus=False)
    # a clamp at dt_min >= 0 makes every step non-negative: accepted, and right
    # (rounded to bf16, so that both sides see the same raw dt)
    small = torch.from_numpy(np.abs(inp.dt) * 0.05).to(torch.bfloat16).to(torch.float64)
    inp.dt = small.numpy().astype(inp.dt.dtype)
    inp.dt_bias = np.zeros_like(inp.dt_bias)
    ref = oracle_run(inp, dt_softplus=False, dt_limit=(0.0, 0.04), input_dt=True)
    y, fin = run_fwd(w, inp, "fused", dt_softplus=False, dt_limit=(0.0, 0.04))
    assert err(y, ref.y) <= TOL_BF16_DESIGN


def test_fused_nemotron_dims_sampled_group():
    # full Nemotron-Nano dims in the benchmark's layout; the oracle runs one
    # group's 8 heads
    w = WORKLOADS["nemotron"]
    inp = make_inputs(w)
    dev = device_inputs(inp, torch.bfloat16, packed_xbc=True)
    out, fin = ssd.ssd_forward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"],
                               dev["dt_bias"], dev["D"], dev["z"], chunk_size=w.chunk_size,
                               out_dtype=torch.bfloat16, algo="fused", input_dt=True)
    torch.cuda.synchronize()
    grp, hpg = 5, w.nheads // w.ngroups
    heads = list(range(grp * hpg, (grp + 1) * hpg))
    sub = head_slice(inp, heads)
    ref = oracle.ssd_fwd(sub.x, sub.B[:, :, grp:grp + 1], sub.C[:, :, grp:grp + 1], sub.dt,
                         sub.A, sub.dt_bias, sub.D, sub.z, threads=8, input_dt=True)
    okay, excess = bf16_out_ok(to_np(out[:, :, heads]), ref.y, TOL_BF16_DESIGN)
    assert okay, excess
    assert err(to_np(fin[:, heads]), ref.final_states) <= TOL_BF16_DESIGN


NAMES = ("dx", "dB", "dC", "ddt", "dA", "ddt_bias", "dD", "dz", "dinitial_states")


@pytest.mark.parametrize("name,decay", [("f32_ragged", None), ("packed", None),
                                        ("bf16_c32", None), ("f32_ragged", -1e4)])
def test_backward(name, decay):
    w = CASES[name]
    inp = with_initial_states(make_inputs(w))
    if decay is not None:
        inp.A = np.full_like(inp.A, decay)
    rng = np.random.default_rng(5)
    dout = rng.standard_normal(inp.x.shape)
    nseq = len(inp.cu_seqlens) - 1 if inp.cu_seqlens is not None else inp.x.shape[0]
    dfin = rng.standard_normal((nseq, w.nheads, w.headdim, w.dstate))
    ref = oracle.ssd_bwd(inp.x, inp.B, inp.C, inp.dt, inp.A, dout, dt_bias=inp.dt_bias,
                         D=inp.D, z=inp.z, initial_states=inp.initial_states,
                         dfinal_states=dfin, cu_seqlens=inp.cu_seqlens, input_dt=True)
    dev = device_inputs(inp, in_dtype(w))
    g = ssd.ssd_backward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"],
                         to_dev(dout, torch.float32), dt_bias=dev["dt_bias"], D=dev["D"],
                         z=dev["z"], initial_states=dev["initial_states"],
                         dfinal_states=to_dev(dfin, torch.float32),
                         cu_seqlens=dev["cu_seqlens"], chunk_size=w.chunk_size, input_dt=True)
    torch.cuda.synchronize()
    errs = {n: err(to_np(getattr(g, n)), getattr(ref, n)) for n in NAMES}
    print({n: f"{e:.2e}" for n, e in errs.items()})
    tol = TOL_F32 if w.dtype == "f32" else TOL_BF16_DESIGN
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{bad} (all: {errs})"
