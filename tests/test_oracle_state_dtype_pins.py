"""Pins of the stored-state forward oracle (``oracle.ssd_fwd_stored_states``)
and of its bf16 rounding (``oracle.round_to_bf16``).

With bf16 state storage the chunked forward no longer reaches the plain
recurrence's result, so its oracle takes the chunked algorithm's steps and
rounds where a state is stored (vLLM PR 27299 "Purpose": the state dtype).  It
is pinned by:
* the rounding itself against torch's float32 -> bfloat16 conversion (a library
  routine), ties and the edges of the range included;
* a hand-derived three-chunk example (``tests/golden``) whose values separate
  rounding the chunk states, rounding the carry-in states, rounding the final
  state and the tie rule;
* exactness: when every stored state is representable, the result is the
  plain recurrence's, bit for bit;
* float32 storage stays within float32 rounding of the plain recurrence;
* packed sequences equal their sequences run one by one.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_round_to_bf16_matches_library_conversion():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact ties: float32 values whose low 16 bits are 0x8000
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32).astype(np.float64),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, -1e-40, 1e-45]),
    ])
    mine = oracle.round_to_bf16(v)
    lib = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(mine, lib)
    assert np.isnan(oracle.round_to_bf16(np.array([np.nan]))[0])
    assert oracle.round_to_bf16(np.array([np.inf]))[0] == np.inf


def _golden():
    d = json.load(open(os.path.join(GOLDEN, "stored_states_bf16_three_chunks.json")))
    sh = lambda v: np.asarray(v, dtype=np.float64).reshape(1, 3, 1, 1)
    args = (sh(d["x"]), sh(d["B"]), sh(d["C"]), np.asarray(d["dt"]).reshape(1, 3, 1), d["A"])
    return d, args


def test_golden_three_chunks_bf16_states():
    d, args = _golden()
    r = oracle.ssd_fwd_stored_states(*args, chunk_size=d["chunk_size"], dt_softplus=False,
                                     state_dtype="bf16")
    assert np.array_equal(r.y.ravel(), np.asarray(d["y_bf16_states"]))
    assert r.final_states.ravel()[0] == d["final_state_bf16_states"]
    # the plain recurrence on the same inputs gives the unrounded values
    p = oracle.ssd_fwd(*args, dt_softplus=False)
    assert np.array_equal(p.y.ravel(), np.asarray(d["y_plain"]))
    assert p.final_states.ravel()[0] == d["final_state_plain"]


def test_exact_when_every_stored_state_is_representable():
    # A = 0 (decay 1), small integer inputs: every state is an integer below
    # 2^8, so storing it in bf16 changes nothing
    rng = np.random.default_rng(5)
    b, T, H, P, N, G = 2, 40, 4, 3, 2, 2
    x = rng.integers(-1, 2, (b, T, H, P)).astype(np.float64)
    B = rng.integers(-1, 2, (b, T, G, N)).astype(np.float64)
    C = rng.integers(-2, 3, (b, T, G, N)).astype(np.float64)
    dt = np.zeros((b, T, H))
    D = rng.integers(-2, 3, H).astype(np.float64)
    h0 = rng.integers(-3, 4, (b, H, P, N)).astype(np.float64)
    p = oracle.ssd_fwd(x, B, C, dt, np.zeros(H), D=D, initial_states=h0, dt_softplus=False)
    for Cs in (4, 7, 64):
        r = oracle.ssd_fwd_stored_states(x, B, C, dt, np.zeros(H), D=D, initial_states=h0,
                                         chunk_size=Cs, dt_softplus=False, state_dtype="bf16")
        assert np.array_equal(r.y, p.y)
        assert np.array_equal(r.final_states, p.final_states)


def test_f32_storage_is_the_plain_recurrence_to_f32_rounding():
    rng = np.random.default_rng(6)
    b, T, H, P, N, G = 1, 77, 4, 3, 5, 2
    x = rng.standard_normal((b, T, H, P)); B = rng.standard_normal((b, T, G, N))
    C = rng.standard_normal((b, T, G, N)); dt = rng.standard_normal((b, T, H))
    A = -np.exp(rng.uniform(-1, 1, H)); bias = rng.uniform(-3, 0, H)
    z = rng.standard_normal((b, T, H, P)); D = rng.standard_normal(H)
    p = oracle.ssd_fwd(x, B, C, dt, A, dt_bias=bias, D=D, z=z)
    r = oracle.ssd_fwd_stored_states(x, B, C, dt, A, dt_bias=bias, D=D, z=z, chunk_size=16,
                                     state_dtype="f32")
    scale = np.sqrt(np.mean(p.y ** 2))
    assert np.max(np.abs(r.y - p.y)) / scale < 1e-6
    assert np.max(np.abs(r.y - p.y)) / scale > 0.0   # it did round
    rb = oracle.ssd_fwd_stored_states(x, B, C, dt, A, dt_bias=bias, D=D, z=z, chunk_size=16,
                                      state_dtype="bf16")
    e = np.max(np.abs(rb.y - p.y)) / scale
    assert 1e-5 < e < 5e-2    # bf16 storage: about 2^-9 of the states' readout


def test_packed_equals_sequences_one_by_one():
    rng = np.random.default_rng(7)
    lens = [9, 0, 21, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, P, N = int(cu[-1]), 2, 3, 4
    x = rng.standard_normal((T, H, P)); B = rng.standard_normal((T, 1, N))
    C = rng.standard_normal((T, 1, N)); dt = rng.standard_normal((T, H))
    A = -np.exp(rng.uniform(-1, 1, H)); h0 = rng.standard_normal((4, H, P, N))
    r = oracle.ssd_fwd_stored_states(x, B, C, dt, A, initial_states=h0, cu_seqlens=cu,
                                     chunk_size=4)
    for i in range(4):
        s, e = int(cu[i]), int(cu[i + 1])
        one = oracle.ssd_fwd_stored_states(x[None, s:e], B[None, s:e], C[None, s:e],
                                           dt[None, s:e], A, initial_states=h0[i:i + 1],
                                           chunk_size=4)
        assert np.array_equal(one.y[0], r.y[s:e])
        assert np.array_equal(one.final_states[0], r.final_states[i])
