"""Shared test helpers: the error metric, device marshalling, oracle runs.

err(gpu, ref) = max_i |gpu_i - ref_i| / sqrt(mean_i ref_i^2), the max error
normalised by the reference's RMS, computed over a whole tensor.

Gates (the forward pass, against the fp64 oracle):
  * fp32 inputs:                         err <= 1e-4
  * bf16 inputs, fp32 output:            err <= 1e-2  (the stated gate); the
    design (hi/lo split of every fp32-derived matrix operand, fp32 states)
    also promises err <= 2e-3, checked as a regression bound
  * bf16 output: |gpu_i - ref_i| <= 1e-2 RMS(ref) + 2^-8 |ref_i| per element,
    i.e. the fp32 gate plus at most one bf16 rounding of the result (a round
    to nearest moves a value by at most 2^-9 of its binade, below 2^-8 |v|).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from mamba_ssd_chunked_scan_amd.inputs import Inputs, Workload, make_inputs

TOL_F32 = 1e-4
TOL_BF16 = 1e-2
TOL_BF16_DESIGN = 2e-3


def err(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r))
    if rms == 0.0:
        return float(np.max(np.abs(g - r))) if g.size else 0.0
    return float(np.max(np.abs(g - r)) / rms) if g.size else 0.0


def bf16_out_ok(gpu, ref, tol=TOL_BF16) -> tuple[bool, float]:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r))
    bound = tol * rms + 2.0 ** -8 * np.abs(r)
    excess = np.max(np.abs(g - r) - bound) if g.size else -1.0
    return bool(excess <= 0.0), float(excess)


def to_dev(a, dtype, device="cuda"):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=dtype)


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def in_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def device_inputs(inp: Inputs, dtype, packed_xbc=False, device="cuda"):
    """Upload x, B, C, dt, z in `dtype`, A, dt_bias, D in float32.

    With packed_xbc, x, B and C are views into one (.., T, H*P + 2*G*N) buffer,
    the production layout where a single projection produces all three.
    """
    x, B, C = inp.x, inp.B, inp.C
    d = {}
    if packed_xbc:
        lead = x.shape[:-2]
        H, P = x.shape[-2:]
        G, N = B.shape[-2:]
        buf = np.concatenate([x.reshape(lead + (H * P,)), B.reshape(lead + (G * N,)),
                              C.reshape(lead + (G * N,))], axis=-1)
        tb = to_dev(buf, dtype, device)
        d["xbc"] = tb
        d["x"] = tb[..., :H * P].unflatten(-1, (H, P))
        d["B"] = tb[..., H * P:H * P + G * N].unflatten(-1, (G, N))
        d["C"] = tb[..., H * P + G * N:].unflatten(-1, (G, N))
    else:
        d["x"], d["B"], d["C"] = to_dev(x, dtype, device), to_dev(B, dtype, device), to_dev(C, dtype, device)
    d["dt"] = to_dev(inp.dt, dtype, device)
    d["z"] = to_dev(inp.z, dtype, device)
    d["A"] = to_dev(inp.A, torch.float32, device)
    d["dt_bias"] = to_dev(inp.dt_bias, torch.float32, device)
    d["D"] = to_dev(inp.D, torch.float32, device)
    d["cu_seqlens"] = (torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device)
                       if inp.cu_seqlens is not None else None)
    d["initial_states"] = to_dev(inp.initial_states, torch.float32, device)
    return d


def oracle_run(inp: Inputs, chunk_size=0, dt_limit=None, dt_softplus=True, threads=None,
               input_dt=False):
    return oracle.ssd_fwd(inp.x, inp.B, inp.C, inp.dt, inp.A, inp.dt_bias, inp.D, inp.z,
                          inp.initial_states, cu_seqlens=inp.cu_seqlens, dt_softplus=dt_softplus,
                          dt_limit=dt_limit, chunk_size=chunk_size, threads=threads,
                          input_dt=input_dt)


def oracle_stored_states_run(inp: Inputs, chunk_size, state_dtype="bf16", threads=None):
    """The chunked forward with its per-chunk states stored in ``state_dtype``."""
    return oracle.ssd_fwd_stored_states(inp.x, inp.B, inp.C, inp.dt, inp.A, inp.dt_bias, inp.D,
                                        inp.z, inp.initial_states, cu_seqlens=inp.cu_seqlens,
                                        chunk_size=chunk_size, state_dtype=state_dtype,
                                        threads=threads)


def stored_state_allowance(inp: Inputs, chunk_size):
    """Per-element allowance of a result whose per-chunk states are stored in bf16.

    A stored state is a rounding of a computed one; the GPU computes its chunk
    states in fp32 where the oracle does fp64, so a value within that small
    difference of a bf16 rounding boundary lands on the other neighbour: one
    bf16 step, at most 2^-7 of its size (8 significant bits).  Such a step in
    a stored chunk state travels through the inter-chunk recurrence, and the
    stored carry-in adds a step of its own, so a stored carry-in can differ by
    at most 2^-7 of the carry built from |S_j| and |h0| (the same recurrence
    on magnitudes, M_j) plus 2^-7 |Hin_j| <= 2^-7 M_j.  Its readout then
    moves an output by at most 2^-6 exp(cs_l) sum_n |C_ln| M_j[p, n] (times
    |silu(z)| when gated).  The final state is not stored in bf16: only the
    chunk-state steps reach it, 2^-7 M_final.  Returns (per-output allowance
    shaped like y, per-final-state allowance).
    """
    x = np.asarray(inp.x, dtype=np.float64)
    packed = inp.cu_seqlens is not None
    lead = 1 if packed else 2
    pk = lambda a: None if a is None else np.asarray(a, np.float64).reshape((-1,) + a.shape[lead:])
    xs, Bs, Cs, dts, zs = pk(x), pk(inp.B), pk(inp.C), pk(inp.dt), pk(inp.z)
    cu = (np.asarray(inp.cu_seqlens, np.int64) if packed
          else np.arange(x.shape[0] + 1, dtype=np.int64) * x.shape[1])
    meta = oracle.varlen_chunk_meta(cu, chunk_size)
    S = oracle.chunk_states(xs, Bs, dts, inp.A, meta, dt_bias=inp.dt_bias)
    cs = oracle.chunk_cumsum(dts, inp.A, meta, chunk_size, dt_bias=inp.dt_bias)
    h0 = None if inp.initial_states is None else np.abs(inp.initial_states)
    M, Mfin = oracle.state_passing(np.abs(oracle.round_to_bf16(S)), cs, meta, h0)
    ry = np.zeros_like(xs)
    if meta.nchunks:
        starts = [meta.start[j] for j in range(meta.nchunks)]
        cut = np.asarray(starts + [meta.start[-1] + meta.length[-1]], dtype=np.int64)
        lo, hi = int(cut[0]), int(cut[-1])
        r = oracle.ssd_fwd(np.zeros_like(xs[lo:hi]), Bs[lo:hi], np.abs(Cs[lo:hi]), dts[lo:hi],
                           inp.A, dt_bias=inp.dt_bias, initial_states=M, cu_seqlens=cut - lo)
        ry[lo:hi] = np.abs(r.y)
    if zs is not None:
        ry = ry * np.abs(zs / (1.0 + np.exp(-zs)))
    return 2.0 ** -6 * ry.reshape(x.shape), 2.0 ** -7 * Mfin


def small_workload(name="small", batch=1, seqlen=300, nheads=4, headdim=32, ngroups=2,
                   dstate=32, chunk_size=64, dtype="bf16", has_D=True, has_z=True, seed=5,
                   nseq=0, seqlens=None):
    return Workload(name, batch, seqlen, nheads, headdim, ngroups, dstate, chunk_size,
                    dtype=dtype, has_D=has_D, has_z=has_z, seed=seed, nseq=nseq,
                    seqlens=seqlens)


def with_initial_states(inp: Inputs, seed=99, scale=1.0) -> Inputs:
    rng = np.random.default_rng(seed)
    H, P = inp.x.shape[-2:]
    N = inp.B.shape[-1]
    nseq = (len(inp.cu_seqlens) - 1) if inp.cu_seqlens is not None else inp.x.shape[0]
    inp.initial_states = (scale * rng.standard_normal((nseq, H, P, N))).astype(np.float32)
    return inp


def head_slice(inp: Inputs, heads, packed=False) -> Inputs:
    """The inputs of a subset of heads (with their groups), for the oracle."""
    H = inp.x.shape[-2]
    G = inp.B.shape[-2]
    hpg = H // G
    heads = list(heads)
    groups = [h // hpg for h in heads]
    ax = 1 if packed else 2
    take = lambda a, idx, axis: None if a is None else np.take(a, idx, axis=axis)
    x = take(inp.x, heads, ax)
    z = take(inp.z, heads, ax)
    dt = take(inp.dt, heads, ax)
    B = take(inp.B, groups, ax)
    C = take(inp.C, groups, ax)
    h0 = None if inp.initial_states is None else inp.initial_states[:, heads]
    return Inputs(x, B, C, dt, inp.A[heads], inp.dt_bias[heads],
                  None if inp.D is None else inp.D[heads], z, inp.cu_seqlens, h0)


__all__ = ["err", "bf16_out_ok", "to_dev", "to_np", "device_inputs", "oracle_run",
           "oracle_stored_states_run", "stored_state_allowance",
           "small_workload", "make_inputs", "with_initial_states", "head_slice", "in_dtype",
           "TOL_F32", "TOL_BF16", "TOL_BF16_DESIGN"]
