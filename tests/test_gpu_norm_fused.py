"""The forward with the gated RMSNorm fused in (ssd_forward_gated_norm) against
the fp64 oracles: the scan (oracle.ssd_fwd, ungated) followed by the gated
RMSNorm (oracle.gated_rmsnorm_fwd, gate first).

Gates: the forward's (bf16 inputs: fp32 output within the design bound 2e-3 of
the output RMS).  A bf16 output is rounded twice on this path -- g when the
scan's epilogue stores it, then the scaled result -- and a round to nearest
moves a bf16 value by up to 2^-8 of itself (half a unit in the last of 8
significant bits, just above a power of two), so per element the bound is the
fp32 gate plus 2 x 2^-8 |ref|.  (ssd_forward followed by ssd_gated_rmsnorm_fwd
rounds twice as well: y, then out.)  The group factors (rstd) are compared
like the fp32 output.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (TOL_BF16_DESIGN, device_inputs, err, head_slice,
                     make_inputs, small_workload, to_np, with_initial_states)
from mamba_ssd_chunked_scan_amd import ssd
from mamba_ssd_chunked_scan_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu


def weight_for(H, P, seed=3):
    rng = np.random.default_rng(seed)
    return (1.0 + 0.3 * rng.standard_normal(H * P)).astype(np.float32)


def reference(inp, w, gs, eps=1e-5, threads=None):
    y = oracle.ssd_fwd(inp.x, inp.B, inp.C, inp.dt, inp.A, inp.dt_bias, inp.D, None,
                       inp.initial_states, cu_seqlens=inp.cu_seqlens, threads=threads)
    n = oracle.gated_rmsnorm_fwd(y.y, inp.z, w, gs, eps)
    return n, y.final_states


def run(inp, w, gs, out_dtype=torch.float32, packed_xbc=False, eps=1e-5):
    dev = device_inputs(inp, torch.bfloat16, packed_xbc=packed_xbc)
    wt = torch.from_numpy(w).cuda()
    lead = dev["x"].shape[:-2]
    W = dev["x"].shape[-2] * dev["x"].shape[-1]
    rstd = torch.empty(int(np.prod(lead)) * (W // gs), dtype=torch.float32, device="cuda")
    out, fin = ssd.ssd_forward_gated_norm(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"], wt,
                                          gs, dev["dt_bias"], dev["D"], dev["z"],
                                          dev["initial_states"], cu_seqlens=dev["cu_seqlens"],
                                          eps=eps, out_dtype=out_dtype, rstd=rstd)
    torch.cuda.synchronize()
    return out, fin, rstd


def twice_rounded_ok(gpu, ref):
    """|gpu - ref| <= 2e-3 RMS(ref) + 2 * 2^-8 |ref| for every element."""
    rms = np.sqrt(np.mean(ref * ref))
    excess = np.max(np.abs(gpu - ref) - (TOL_BF16_DESIGN * rms + 2.0 ** -7 * np.abs(ref)))
    return bool(excess <= 0.0), float(excess)


def check(out, fin, rstd, ref, ref_fin, out_dtype):
    go = to_np(out)
    if out_dtype == torch.float32:
        e = err(go, ref.out)
        assert e <= TOL_BF16_DESIGN, f"output err {e:.3e}"
    else:
        okay, excess = twice_rounded_ok(go, ref.out)
        assert okay, f"bf16 output exceeds its bound by {excess:.3e}"
    er = err(to_np(rstd), ref.rstd.reshape(-1))
    assert er <= TOL_BF16_DESIGN, f"rstd err {er:.3e}"
    ef = err(to_np(fin), ref_fin)
    assert ef <= TOL_BF16_DESIGN, f"final state err {ef:.3e}"


CASES = {
    "groups_of_one_head": (dict(batch=2, seqlen=333, nheads=8, headdim=64, ngroups=2, dstate=64,
                                chunk_size=64), 64),
    "groups_of_8_heads": (dict(seqlen=700, nheads=16, headdim=64, ngroups=2, dstate=128,
                               chunk_size=128), 512),
    "one_group_all_heads": (dict(seqlen=400, nheads=4, headdim=128, ngroups=1, dstate=32,
                                 chunk_size=128), 512),
    "packed": (dict(seqlen=1500, nheads=8, headdim=64, ngroups=4, dstate=64, chunk_size=64,
                    seqlens=(500, 0, 1, 999)), 128),
    "no_gate": (dict(seqlen=300, nheads=8, headdim=64, ngroups=2, dstate=64, chunk_size=64,
                     has_z=False), 256),
}


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("name", sorted(CASES))
def test_small_every_element(name, out_dtype):
    kw, gs = CASES[name]
    w_ = small_workload(name, **kw)
    inp = with_initial_states(make_inputs(w_))
    w = weight_for(w_.nheads, w_.headdim)
    ref, ref_fin = reference(inp, w, gs)
    out, fin, rstd = run(inp, w, gs, out_dtype)
    check(out, fin, rstd, ref, ref_fin, out_dtype)


def test_matches_the_two_call_path():
    # ssd_forward (ungated, fp32 out) then ssd_gated_rmsnorm_fwd: the same
    # function in two passes, agreeing to their rounding
    kw, gs = CASES["groups_of_8_heads"]
    w_ = small_workload("two_call", **kw)
    inp = with_initial_states(make_inputs(w_))
    w = weight_for(w_.nheads, w_.headdim)
    out, fin, rstd = run(inp, w, gs)
    dev = device_inputs(inp, torch.bfloat16)
    y, _ = ssd.ssd_forward(dev["x"], dev["B"], dev["C"], dev["dt"], dev["A"], dev["dt_bias"],
                           dev["D"], None, dev["initial_states"], chunk_size=128,
                           out_dtype=torch.float32, algo="fused")
    ref2, _ = ssd.ssd_gated_rmsnorm_fwd(y, dev["z"].float(), torch.from_numpy(w).cuda(), gs)
    torch.cuda.synchronize()
    assert err(to_np(out), to_np(ref2)) <= 1e-4


@pytest.mark.parametrize("name,gs,ngroups_sampled", [("nemotron", 512, 2), ("granite", 8192, 0)])
def test_full_size(name, gs, ngroups_sampled):
    # benchmark launch configuration (x/B/C views of one xBC buffer); Nemotron-Nano's
    # norm groups are 8 heads: two whole groups sampled; Granite's one group
    # spans every head: the whole output
    w_ = WORKLOADS[name]
    inp = make_inputs(w_)
    w = weight_for(w_.nheads, w_.headdim)
    out, fin, rstd = run(inp, w, gs, torch.bfloat16, packed_xbc=True)
    go = to_np(out)
    assert np.all(np.isfinite(go))
    hpg = gs // w_.headdim
    if ngroups_sampled:
        groups = [0, (w_.nheads // hpg) - 1][:ngroups_sampled]
        heads = [g * hpg + k for g in groups for k in range(hpg)]
        sub = head_slice(inp, heads)
        ref, ref_fin = reference(sub, w.reshape(w_.nheads, -1)[heads].reshape(-1), gs,
                                 threads=16)
        got = np.take(go, heads, axis=2)
        got_r = to_np(rstd).reshape(w_.seqlen, -1)[:, groups]
        got_f = to_np(fin)[:, heads]
    else:
        ref, ref_fin = reference(inp, w, gs, threads=16)
        got, got_r, got_f = go, to_np(rstd).reshape(w_.seqlen, -1), to_np(fin)
    okay, excess = twice_rounded_ok(got, ref.out)
    assert okay, f"bf16 output exceeds its bound by {excess:.3e}"
    assert err(got_r, ref.rstd.reshape(got_r.shape)) <= TOL_BF16_DESIGN
    assert err(got_f, ref_fin) <= TOL_BF16_DESIGN
    # bitwise repeatable
    out2, fin2, _ = run(inp, w, gs, torch.bfloat16, packed_xbc=True)
    assert torch.equal(out, out2) and torch.equal(fin, fin2)


def test_rejects_what_it_does_not_take():
    w_ = small_workload("p32", seqlen=64, nheads=4, headdim=32, ngroups=1, dstate=32,
                        chunk_size=64)
    inp = make_inputs(w_)
    with pytest.raises(ssd.SSDError) as e:
        run(inp, weight_for(4, 32), 64)
    assert e.value.status == 5          # headdim not a multiple of 64
    w_ = small_workload("gs96", seqlen=64, nheads=3, headdim=64, ngroups=1, dstate=32,
                        chunk_size=64)
    inp = make_inputs(w_)
    with pytest.raises(ssd.SSDError) as e:
        run(inp, weight_for(3, 64), 96)
    assert e.value.status == 2          # group_size not a multiple of 64
