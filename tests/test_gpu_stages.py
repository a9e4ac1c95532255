"""Per-stage parity of the HIP kernels against the fp64 oracle.

Each stage is fed the ORACLE's intermediates (cumsum, CB, chunk states,
carry-in states), cast to what the C ABI takes, so a mismatch points at the
stage that produced it.  All calls go through the C ABI (ctypes binding).
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_chunked_scan_amd import ssd
from helpers import (TOL_BF16, TOL_BF16_DESIGN, TOL_F32, device_inputs, err, in_dtype,
                     make_inputs, oracle_run, small_workload, to_dev, to_np,
                     with_initial_states)

pytestmark = pytest.mark.gpu

CASES = {
    # name: workload; shapes span several tiles and a ragged last chunk
    "f32_tiny": small_workload("f32_tiny", seqlen=256, nheads=4, headdim=16, ngroups=1,
                               dstate=16, chunk_size=64, dtype="f32", has_z=False),
    "bf16_ragged": small_workload("bf16_ragged", batch=2, seqlen=300, nheads=6, headdim=32,
                                  ngroups=2, dstate=48, chunk_size=64),
    "bf16_c128": small_workload("bf16_c128", seqlen=520, nheads=4, headdim=64, ngroups=1,
                                dstate=128, chunk_size=128),
    "f32_c32_ragged": small_workload("f32_c32_ragged", seqlen=77, nheads=3, headdim=16,
                                     ngroups=3, dstate=32, chunk_size=32, dtype="f32"),
    "bf16_c256_p128": small_workload("bf16_c256_p128", seqlen=600, nheads=2, headdim=128,
                                     ngroups=1, dstate=64, chunk_size=256),
    "packed": small_workload("packed", seqlen=700, nheads=4, headdim=32, ngroups=2,
                             dstate=32, chunk_size=64, seqlens=(1, 63, 64, 65, 0, 200, 307)),
}


def tol_of(w):
    return TOL_F32 if w.dtype == "f32" else TOL_BF16_DESIGN


def setup(name):
    w = CASES[name]
    inp = with_initial_states(make_inputs(w))
    dev = device_inputs(inp, in_dtype(w))
    packed = inp.cu_seqlens is not None
    prob = ssd.problem_from(dev["x"], dev["B"], w.chunk_size, cu_seqlens=dev["cu_seqlens"])
    if packed:
        prob.chunk_meta = ssd.ssd_varlen_chunk_meta(prob)
        meta = oracle.varlen_chunk_meta(inp.cu_seqlens, w.chunk_size)
        tok = lambda a: a
    else:
        meta = oracle.batch_chunk_meta(w.batch, w.seqlen, w.chunk_size)
        tok = lambda a: None if a is None else a.reshape((-1,) + a.shape[2:])
    return w, inp, dev, prob, meta, tok


def valid_cs(cs, meta):
    """Entries of a (K, H, C) tensor that belong to real chunks."""
    return cs[:meta.nchunks]


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_cumsum(name):
    w, inp, dev, prob, meta, tok = setup(name)
    got = ssd.ssd_chunk_cumsum(prob, dev["dt"], dev["A"], dev["dt_bias"])
    torch.cuda.synchronize()
    ref = oracle.chunk_cumsum(tok(inp.dt), inp.A, meta, w.chunk_size, dt_bias=inp.dt_bias)
    e = err(valid_cs(to_np(got), meta), ref)
    assert e <= 1e-5, e


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_cumsum_dt_out_and_clamp(name):
    w, inp, dev, prob, meta, tok = setup(name)
    prob.dt_limit = (0.01, 0.05)
    K = prob.num_chunks()
    dt_out = torch.empty((K, w.nheads, w.chunk_size), dtype=torch.float32, device="cuda")
    got = ssd.ssd_chunk_cumsum(prob, dev["dt"], dev["A"], dev["dt_bias"], dt_out=dt_out)
    torch.cuda.synchronize()
    lim = (np.float64(np.float32(0.01)), np.float64(np.float32(0.05)))
    ref = oracle.chunk_cumsum(tok(inp.dt), inp.A, meta, w.chunk_size, dt_bias=inp.dt_bias,
                              dt_limit=lim)
    assert err(valid_cs(to_np(got), meta), ref) <= 1e-5
    d = to_np(dt_out)[:meta.nchunks]
    step = oracle.step_size(tok(inp.dt), inp.dt_bias, dt_limit=lim)
    for j in range(meta.nchunks):
        s, L = meta.start[j], meta.length[j]
        np.testing.assert_allclose(d[j, :, :L].T, step[s:s + L], rtol=1e-6, atol=0)
        assert np.all(d[j, :, L:] == 0.0)


@pytest.mark.parametrize("name", sorted(CASES))
def test_bmm_chunk(name):
    w, inp, dev, prob, meta, tok = setup(name)
    got = to_np(ssd.ssd_bmm_chunk(prob, dev["C"], dev["B"]))
    torch.cuda.synchronize()
    ref = oracle.bmm_chunk(tok(inp.C), tok(inp.B), meta, w.chunk_size)
    mask = np.tril(np.ones((w.chunk_size, w.chunk_size), dtype=bool))
    g = got[:meta.nchunks][..., mask]
    r = ref[..., mask]
    # rows/cols past a short chunk's end are zero in the reference and must be
    # finite (they are never read) -- compare only the real ones
    for j in range(meta.nchunks):
        L = meta.length[j]
        blk = got[j][:, :L, :L][:, mask[:L, :L]]
        rblk = ref[j][:, :L, :L][:, mask[:L, :L]]
        np.testing.assert_allclose(blk, rblk, rtol=2e-6, atol=2e-6 * np.sqrt(w.dstate))
    assert err(g, r) <= 1e-5


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_chunk_state(name, state_dtype):
    w, inp, dev, prob, meta, tok = setup(name)
    prob.state_dtype = state_dtype
    cs_ref = oracle.chunk_cumsum(tok(inp.dt), inp.A, meta, w.chunk_size, dt_bias=inp.dt_bias)
    cs = torch.zeros((prob.num_chunks(), w.nheads, w.chunk_size), dtype=torch.float32,
                     device="cuda")
    cs[:meta.nchunks] = to_dev(cs_ref, torch.float32)
    got = to_np(ssd.ssd_chunk_state(prob, dev["x"], dev["B"], cs))[:meta.nchunks]
    torch.cuda.synchronize()
    ref = oracle.chunk_states(tok(inp.x), tok(inp.B), tok(inp.dt), inp.A, meta,
                              dt_bias=inp.dt_bias)
    if state_dtype == torch.bfloat16:
        # one bf16 rounding of the stored state: <= 2^-8 |v| per element
        bound = tol_of(w) * np.sqrt(np.mean(ref ** 2)) + 2.0 ** -8 * np.abs(ref)
        assert np.all(np.abs(got - ref) <= bound)
    else:
        assert err(got, ref) <= tol_of(w)


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_state_passing(name, state_dtype):
    w, inp, dev, prob, meta, tok = setup(name)
    prob.state_dtype = state_dtype
    S = oracle.chunk_states(tok(inp.x), tok(inp.B), tok(inp.dt), inp.A, meta,
                            dt_bias=inp.dt_bias)
    cs_ref = oracle.chunk_cumsum(tok(inp.dt), inp.A, meta, w.chunk_size, dt_bias=inp.dt_bias)
    K = prob.num_chunks()
    cs = torch.zeros((K, w.nheads, w.chunk_size), dtype=torch.float32, device="cuda")
    cs[:meta.nchunks] = to_dev(cs_ref, torch.float32)
    st = torch.zeros((K, w.nheads, w.headdim, w.dstate), dtype=state_dtype, device="cuda")
    st[:meta.nchunks] = to_dev(S, state_dtype)
    # both sides see the same (stored, possibly rounded) chunk states and cumsum
    S_in = to_np(st)[:meta.nchunks]
    cs_in = to_np(cs)[:meta.nchunks]
    ref_in, ref_fin = oracle.state_passing(S_in, cs_in, meta, inp.initial_states)
    h0 = to_dev(inp.initial_states, torch.float32)
    hin, fin = ssd.ssd_state_passing(prob, st, cs, initial_states=h0, states_out=st)  # in place
    torch.cuda.synchronize()
    got_in = to_np(hin)[:meta.nchunks]
    assert err(to_np(fin), ref_fin) <= TOL_F32
    if state_dtype == torch.float32:
        assert err(got_in, ref_in) <= TOL_F32
    else:
        # fp32 recurrence, one bf16 rounding when stored
        bound = TOL_F32 * np.sqrt(np.mean(ref_in ** 2)) + 2.0 ** -8 * np.abs(ref_in)
        assert np.all(np.abs(got_in - ref_in) <= bound)


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_chunk_scan(name, out_dtype):
    w, inp, dev, prob, meta, tok = setup(name)
    r = oracle_run(inp, chunk_size=w.chunk_size)
    cs_ref = oracle.chunk_cumsum(tok(inp.dt), inp.A, meta, w.chunk_size, dt_bias=inp.dt_bias)
    cb_ref = oracle.bmm_chunk(tok(inp.C), tok(inp.B), meta, w.chunk_size)
    hin_ref = oracle.carry_in_states(r.chunk_end_states, meta, inp.initial_states)
    K = prob.num_chunks()
    cs = torch.zeros((K, w.nheads, w.chunk_size), dtype=torch.float32, device="cuda")
    cs[:meta.nchunks] = to_dev(cs_ref, torch.float32)
    cb = torch.zeros((K, w.ngroups, w.chunk_size, w.chunk_size), dtype=torch.float32,
                     device="cuda")
    cb[:meta.nchunks] = to_dev(cb_ref, torch.float32)
    hin = torch.zeros((K, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")
    hin[:meta.nchunks] = to_dev(hin_ref, torch.float32)
    out = ssd.ssd_chunk_scan(prob, cb, dev["x"], dev["C"], cs, hin, D=dev["D"], z=dev["z"],
                             out_dtype=out_dtype)
    torch.cuda.synchronize()
    got = to_np(out)
    if out_dtype == torch.float32:
        assert err(got, r.y) <= tol_of(w)
    else:
        from helpers import bf16_out_ok
        okay, excess = bf16_out_ok(got, r.y, tol_of(w))
        assert okay, excess


def test_varlen_meta_device_matches_oracle_bit_exact():
    rng = np.random.default_rng(3)
    for trial in range(40):
        nseq = int(rng.integers(1, 40))
        T = int(rng.integers(0, 5000))
        cuts = np.sort(rng.integers(0, T + 1, nseq - 1))
        cu = np.array([0] + [int(v) for v in cuts] + [T], dtype=np.int32)
        C = int(rng.choice([32, 64, 128, 256]))
        if T == 0:
            continue
        p = ssd.Problem(1, T, 4, 16, 1, 16, C, nseq=nseq,
                        cu_seqlens=torch.from_numpy(cu).cuda())
        got = ssd.ssd_varlen_chunk_meta(p).cpu().tolist()
        m = oracle.varlen_chunk_meta(cu, C)
        K = -(-T // C) + nseq
        exp = [m.nchunks, nseq, C, K]
        for j in range(K):
            exp += [m.seq[j], m.start[j], m.length[j]] if j < m.nchunks else [-1, 0, 0]
        exp += m.first_chunk
        assert got == exp, (trial, cu.tolist(), C)
        assert got == ssd.ssd_varlen_chunk_meta_host(p, cu.tolist())
