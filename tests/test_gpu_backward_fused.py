"""The per-chunk backward (ssd_backward_ex with SSD_ALGO_FUSED) against the
fp64 backward oracle (oracle.ssd_bwd) and against the staged backward.

Every gradient is compared with err() = max |gpu - ref| / RMS(ref) over the
whole tensor and held to the forward's bf16 design bound (2e-3): the path
takes bf16 x, B, C only.  The cases cover what the per-chunk kernels
distinguish: ragged last chunks, packed sequences (empty ones, lengths around
the 128-token chunk), d_state below the 16-column tile multiple of the
kernels' n-tiles (48) and at 64 and 128, groups of one to 20 heads (more than
8 heads per group take the head-split partial sums), odd heads per group, no
gate / skip / states, the clamp, no softplus, the step size on the input term,
a bf16 upstream gradient, strong, zero and growing decay, and repeats (bit for
bit).
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_chunked_scan_amd import ssd
from helpers import (TOL_BF16_DESIGN, device_inputs, err, make_inputs, small_workload, to_dev,
                     to_np, with_initial_states)

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


def gpu_bwd(w, inp, dout, dfin, algo, dout_dtype=torch.float32, **kw):
    dev = device_inputs(inp, torch.bfloat16)
    g = ssd.ssd_backward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"],
                         to_dev(dout, dout_dtype), dt_bias=dev["dt_bias"], D=dev["D"],
                         z=dev["z"], initial_states=dev["initial_states"],
                         dfinal_states=to_dev(dfin, torch.float32),
                         cu_seqlens=dev["cu_seqlens"], chunk_size=w.chunk_size, algo=algo, **kw)
    torch.cuda.synchronize()
    return g


def ref_bwd(inp, dout, dfin, dt_limit=None, dt_softplus=True, input_dt=False):
    return oracle.ssd_bwd(inp.x, inp.B, inp.C, inp.dt, inp.A, dout, dt_bias=inp.dt_bias, D=inp.D,
                          z=inp.z, initial_states=inp.initial_states, dfinal_states=dfin,
                          cu_seqlens=inp.cu_seqlens, dt_softplus=dt_softplus, dt_limit=dt_limit,
                          input_dt=input_dt)


def check(g, ref, tol=TOL_BF16_DESIGN, skip=()):
    errs = {}
    for n in NAMES:
        if n in skip:
            continue
        a, r = getattr(g, n), getattr(ref, n)
        if r is None:
            assert a is None, n
            continue
        errs[n] = err(to_np(a), r)
    print({n: f"{e:.2e}" for n, e in errs.items()})
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"gradients over {tol:g}: {bad} (all: {errs})"


def run_case(w, inp, dout, dfin, **kw):
    ref_kw = {k: kw[k] for k in ("dt_limit", "dt_softplus", "input_dt") if k in kw}
    ref = ref_bwd(inp, dout, dfin, **ref_kw)
    g = gpu_bwd(w, inp, dout, dfin, "fused", **kw)
    check(g, ref)
    return g, ref


CASES = {
    # ragged batch rows, two groups of two heads, d_state 128
    "batch_n128": dict(batch=2, seqlen=300, nheads=4, ngroups=2, dstate=128),
    # d_state 64 (the 4-tile kernel) and 48 (columns past N masked)
    "n64_chunk_multiple": dict(batch=1, seqlen=384, nheads=4, ngroups=1, dstate=64),
    "n48_odd_heads": dict(batch=1, seqlen=200, nheads=6, ngroups=2, dstate=48),
    # 20 heads in one group: three head splits of 7, 7, 6 summed by the reduce kernel
    "one_group_20_heads": dict(batch=1, seqlen=260, nheads=20, ngroups=1, dstate=128),
    # one token
    "single_token": dict(batch=1, seqlen=1, nheads=2, ngroups=1, dstate=32),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_cases_against_oracle(name):
    w = small_workload(name, headdim=64, chunk_size=64, **CASES[name])
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    run_case(w, inp, dout, dfin)


VARLEN = (300, 0, 1, 127, 128, 129, 0, 255)


def test_packed_sequences():
    w = small_workload("bwdf_varlen", seqlen=sum(VARLEN), nheads=4, headdim=64, ngroups=2,
                       dstate=64, chunk_size=64, seqlens=VARLEN)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    g, _ = run_case(w, inp, dout, dfin)
    cu = inp.cu_seqlens
    for i in range(len(cu) - 1):
        if cu[i + 1] == cu[i]:  # an empty sequence passes its final-state gradient through
            assert np.array_equal(to_np(g.dinitial_states[i]), dfin[i].astype(np.float32))


def test_no_gate_no_skip_no_states():
    w = small_workload("bwdf_plain", seqlen=257, nheads=2, headdim=64, ngroups=1, dstate=64,
                       chunk_size=128, has_D=False, has_z=False)
    inp = make_inputs(w)
    dout, _ = upstream(inp, dfinal=False)
    run_case(w, inp, dout, None)


def test_clamp():
    w = small_workload("bwdf_clamp", seqlen=200, nheads=6, headdim=64, ngroups=2, dstate=64,
                       chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    delta = oracle.step_size(inp.dt, inp.dt_bias)
    lim = tuple(float(v) for v in np.quantile(delta, [0.2, 0.8]))
    dout, dfin = upstream(inp)
    g, _ = run_case(w, inp, dout, dfin, dt_limit=lim)
    clamped = (delta < lim[0]) | (delta > lim[1])
    assert np.all(to_np(g.ddt)[clamped] == 0.0)


def test_without_softplus():
    w = small_workload("bwdf_nosp", seqlen=150, nheads=2, headdim=64, ngroups=2, dstate=32,
                       chunk_size=64)
    inp = with_initial_states(make_inputs(w))
    small = np.abs(inp.dt) * 0.05 + 0.01
    inp.dt = torch.from_numpy(small).to(torch.bfloat16).to(torch.float64).numpy()
    inp.dt_bias = np.zeros_like(inp.dt_bias)
    dout, dfin = upstream(inp)
    run_case(w, inp, dout, dfin, dt_softplus=False)


def test_input_dt():
    w = small_workload("bwdf_idt", batch=2, seqlen=300, nheads=4, headdim=64, ngroups=2,
                       dstate=128, chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    run_case(w, inp, dout, dfin, input_dt=True)


def test_bf16_upstream_gradient():
    w = small_workload("bwdf_dout16", seqlen=300, nheads=4, headdim=64, ngroups=2, dstate=64,
                       chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    dout = torch.from_numpy(dout).to(torch.bfloat16).to(torch.float64).numpy()
    ref = ref_bwd(inp, dout, dfin)
    g = gpu_bwd(w, inp, dout, dfin, "fused", dout_dtype=torch.bfloat16)
    check(g, ref)


@pytest.mark.parametrize("case", ["strong_decay", "no_decay", "weak_positive"])
def test_decay_rates(case):
    w = small_workload(f"bwdf_{case}", seqlen=190, nheads=4, headdim=64, ngroups=2, dstate=32,
                       chunk_size=64)
    inp = with_initial_states(make_inputs(w))
    inp.A = np.full_like(inp.A, {"strong_decay": -1e4, "no_decay": 0.0, "weak_positive": 0.01}[case])
    dout, dfin = upstream(inp)
    ref = ref_bwd(inp, dout, dfin)
    g = gpu_bwd(w, inp, dout, dfin, "fused")
    if case == "no_decay":
        # A = 0: the raw step gets no gradient (exactly), A still does
        assert np.all(to_np(g.ddt) == 0.0) and np.all(to_np(g.ddt_bias) == 0.0)
        check(g, ref, skip=("ddt", "ddt_bias"))
    else:
        check(g, ref)


def test_agrees_with_staged_and_chunk_size_is_internal():
    w = small_workload("bwdf_vs_staged", batch=2, seqlen=333, nheads=4, headdim=64, ngroups=2,
                       dstate=64, chunk_size=64)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    gf = gpu_bwd(w, inp, dout, dfin, "fused")
    gs = gpu_bwd(w, inp, dout, dfin, "staged")
    for n in NAMES:
        a, b = getattr(gf, n), getattr(gs, n)
        assert err(to_np(a), to_np(b)) <= TOL_BF16_DESIGN, n
    # the per-chunk path always works on 128-token chunks: another chunk_size
    # gives the same bits
    w2 = small_workload("bwdf_vs_staged", batch=2, seqlen=333, nheads=4, headdim=64, ngroups=2,
                        dstate=64, chunk_size=256)
    g2 = gpu_bwd(w2, inp, dout, dfin, "fused")
    for n in NAMES:
        assert torch.equal(getattr(gf, n), getattr(g2, n)), n


def test_auto_routes():
    w = small_workload("bwdf_auto", seqlen=200, nheads=4, headdim=64, ngroups=2, dstate=64,
                       chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    ga = gpu_bwd(w, inp, dout, dfin, "auto")
    gf = gpu_bwd(w, inp, dout, dfin, "fused")
    for n in NAMES:
        assert torch.equal(getattr(ga, n), getattr(gf, n)), n
    prob = ssd.problem_from(torch.empty(1, 200, 4, 64), torch.empty(1, 200, 2, 64), 128)
    assert prob.backward_workspace_size("fused") < prob.backward_workspace_size("staged")
    assert prob.backward_workspace_size("auto") == prob.backward_workspace_size("fused")
    assert (prob.backward_workspace_size("auto", torch.float32)
            == prob.backward_workspace_size("staged"))


def test_rejects_what_it_does_not_take():
    # headdim 32 and fp32 inputs: SSD_ERR_UNSUPPORTED naming the staged path
    w = small_workload("bwdf_rej", seqlen=100, nheads=2, headdim=32, ngroups=1, dstate=32,
                       chunk_size=64)
    inp = make_inputs(w)
    dout, _ = upstream(inp, dfinal=False)
    with pytest.raises(ssd.SSDError, match="STAGED") as e:
        gpu_bwd(w, inp, dout, None, "fused")
    assert e.value.status == 5
    w = small_workload("bwdf_rej32", seqlen=100, nheads=2, headdim=64, ngroups=1, dstate=32,
                       chunk_size=64, dtype="f32")
    inp = make_inputs(w)
    dout, _ = upstream(inp, dfinal=False)
    dev = device_inputs(inp, torch.float32)
    with pytest.raises(ssd.SSDError) as e:
        ssd.ssd_backward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"],
                         to_dev(dout, torch.float32), dt_bias=dev["dt_bias"], D=dev["D"],
                         z=dev["z"], chunk_size=64, algo="fused")
    assert e.value.status == 5


def _equal_grads(a, b):
    for n in NAMES:
        x, y = getattr(a, n), getattr(b, n)
        assert (x is None) == (y is None), n
        if x is not None:
            assert torch.equal(x, y), f"{n} differs between head passes and one pass"


@pytest.mark.parametrize("case", ["whole_groups", "within_a_group", "within_a_group_input_dt"])
def test_head_passes_match_one_pass(case):
    """A smaller workspace makes the backward take its heads in passes: four
    passes of one group (two heads each), or one group of 24 heads in passes of
    16 and 8 (dB and dC summed over the group's passes in split order).  Every
    gradient equals the one-pass result bit for bit; packed sequences with
    initial states and a final-state gradient exercise the state tensors'
    head offsets."""
    if case == "whole_groups":
        H, G, hsmall, gsmall = 8, 4, 2, 1
    else:
        H, G, hsmall, gsmall = 24, 1, 16, 1
    kw = {"input_dt": True} if case.endswith("input_dt") else {}
    lens = (130, 0, 257, 64)
    w = small_workload(f"bwdf_pass_{case}", seqlen=sum(lens), nheads=H, headdim=64, ngroups=G,
                       dstate=64, chunk_size=128, seqlens=lens)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    one = gpu_bwd(w, inp, dout, dfin, "fused", **kw)
    cu = device_inputs(inp, torch.bfloat16)["cu_seqlens"]
    small = ssd.Problem(1, w.seqlen, hsmall, 64, gsmall, 64, 128, nseq=len(lens), cu_seqlens=cu,
                        **kw)
    need = small.backward_workspace_size("fused")
    full = ssd.Problem(1, w.seqlen, H, 64, G, 64, 128, nseq=len(lens), cu_seqlens=cu, **kw)
    assert need < full.backward_workspace_size("fused")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    passes = gpu_bwd(w, inp, dout, dfin, "fused", workspace=ws, **kw)
    _equal_grads(passes, one)
    check(passes, ref_bwd(inp, dout, dfin, **kw))
    # below the smallest pass: an error, nothing launched
    tiny = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(ssd.SSDError):
        gpu_bwd(w, inp, dout, dfin, "fused", workspace=tiny, **kw)


def test_bit_identical_repeats():
    w = small_workload("bwdf_rep", seqlen=700, nheads=16, headdim=64, ngroups=1, dstate=128,
                       chunk_size=128)
    inp = with_initial_states(make_inputs(w))
    dout, dfin = upstream(inp)
    g1 = gpu_bwd(w, inp, dout, dfin, "fused")
    g2 = gpu_bwd(w, inp, dout, dfin, "fused")
    for n in NAMES:
        assert torch.equal(getattr(g1, n), getattr(g2, n)), n


def test_full_size_granite_every_gradient():
    # granite-4.0-h-small dims (4096 tokens, 128 heads x 64 in one group,
    # d_state 128): every gradient of the whole problem against the oracle,
    # dB and dC summed over all 128 heads (16 head splits and their reduction)
    from mamba_ssd_chunked_scan_amd.inputs import WORKLOADS
    w = WORKLOADS["granite"]
    inp = make_inputs(w)
    dout, dfin = upstream(inp, seed=11)
    ref = oracle.ssd_bwd(inp.x, inp.B, inp.C, inp.dt, inp.A, dout, dt_bias=inp.dt_bias, D=inp.D,
                         z=inp.z, dfinal_states=dfin, threads=16)
    g = gpu_bwd(w, inp, dout, dfin, "fused")
    check(g, ref)
