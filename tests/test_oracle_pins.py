"""Pins of the fp64 oracle against facts other than itself.

Each test ties the oracle to something the pages or the mathematics fix:
a hand-derived example, the closed form of the recurrence, special cases
that reduce to library routines, invariants (split/resume, packing, group
expansion, linearity, causality), and a chunked evaluation worked out
here from the recurrence chunk by chunk (the pages' chunkwise decomposition:
intra-chunk outputs, chunk end states, the decay_chunk window of the
inter-chunk propagation, the readout).

A plausible slip in the oracle -- a dropped term, a sign, an index off by
one, transposed operands, the decay applied after instead of before the
update, the wrong group for a head -- fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(rng, b=2, T=23, H=4, P=3, N=5, G=2, gated=True, with_D=True, h0=True):
    x = rng.standard_normal((b, T, H, P))
    B = rng.standard_normal((b, T, G, N))
    C = rng.standard_normal((b, T, G, N))
    dt = rng.standard_normal((b, T, H))
    A = -np.exp(rng.uniform(0.0, np.log(4.0), H))
    bias = rng.uniform(-2.0, 0.5, H)
    D = rng.standard_normal(H) if with_D else None
    z = rng.standard_normal((b, T, H, P)) if gated else None
    init = rng.standard_normal((b, H, P, N)) if h0 else None
    return dict(x=x, B=B, C=C, dt=dt, A=A, dt_bias=bias, D=D, z=z, initial_states=init)


def plain_softplus(u):
    # the textbook definition; fine for the moderate arguments used here
    return np.log(1.0 + np.exp(u))


def closed_form(x, B, C, dt, A, dt_bias, D=None, z=None, initial_states=None, input_dt=False):
    """y_t = sum_{s<=t} C_t^T (prod_{u=s+1..t} abar_u) B_s x_s
           + C_t^T (prod_{u<=t} abar_u) h_init  + D x_t,  then the SiLU gate.

    SSD Reference, section "Math": the closed form with the empty product = 1;
    the initial-state term decays through every token up to t (section
    "Inter-chunk propagation", the init term).  Brute force, O(T^2), explicit
    products of per-token decays (no cumulative sums).  With ``input_dt`` the
    input of token s enters as delta_s x_s (Mamba-2's discretised input);
    the skip still reads x_t.
    """
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros_like(x)
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            delta = plain_softplus(dt[bi, :, h] + dt_bias[h])
            abar = np.exp(delta * A[h])
            for t in range(T):
                acc = np.zeros(P)
                for s in range(t + 1):
                    w = np.prod(abar[s + 1:t + 1])  # empty product is 1
                    if input_dt:
                        w = w * delta[s]
                    acc += w * np.dot(C[bi, t, g], B[bi, s, g]) * x[bi, s, h]
                if initial_states is not None:
                    w0 = np.prod(abar[:t + 1])
                    acc += w0 * (initial_states[bi, h] @ C[bi, t, g])
                if D is not None:
                    acc += D[h] * x[bi, t, h]
                if z is not None:
                    zz = z[bi, t, h]
                    acc = acc * zz / (1.0 + np.exp(-zz))
                y[bi, t, h] = acc
    return y


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- golden

def test_golden_scalar_three_tokens():
    d = json.load(open(os.path.join(GOLDEN, "scalar_three_tokens.json")))
    sh = lambda v: np.asarray(v, dtype=np.float64).reshape(1, 3, 1, 1)
    x, B, C = sh(d["x"]), sh(d["B"]), sh(d["C"])
    dt = np.asarray(d["dt"]).reshape(1, 3, 1)
    r = oracle.ssd_fwd(x, B, C, dt, d["A"], D=d["D"], dt_softplus=d["dt_softplus"])
    np.testing.assert_allclose(r.y.ravel(), d["y"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(r.final_states.ravel(), [d["final_state"]], rtol=1e-15)
    rg = oracle.ssd_fwd(x, B, C, dt, d["A"], D=d["D"], z=sh(d["z"]),
                        dt_softplus=d["dt_softplus"])
    np.testing.assert_allclose(rg.y.ravel(), d["out_gated"], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- closed form

@pytest.mark.parametrize("gated,with_D,h0", [(False, False, False), (True, True, True),
                                             (False, True, True), (True, False, False)])
def test_closed_form(gated, with_D, h0):
    rng = np.random.default_rng(7)
    pr = rand_problem(rng, gated=gated, with_D=with_D, h0=h0)
    r = oracle.ssd_fwd(**pr)
    ref = closed_form(**pr)
    assert rel(r.y, ref) < 1e-12


def test_closed_form_odd_groups_and_long_memory():
    # 6 heads in 2 groups (3 heads per group), slow decay so old tokens matter
    rng = np.random.default_rng(11)
    pr = rand_problem(rng, b=1, T=40, H=6, P=2, N=3, G=2)
    pr["A"] = -np.exp(rng.uniform(np.log(1e-3), np.log(1e-2), 6))
    r = oracle.ssd_fwd(**pr)
    assert rel(r.y, closed_form(**pr)) < 1e-12


@pytest.mark.parametrize("gated,with_D,h0", [(False, False, False), (True, True, True)])
def test_closed_form_input_dt(gated, with_D, h0):
    rng = np.random.default_rng(17)
    pr = rand_problem(rng, gated=gated, with_D=with_D, h0=h0)
    r = oracle.ssd_fwd(**pr, input_dt=True)
    ref = closed_form(**pr, input_dt=True)
    assert rel(r.y, ref) < 1e-12
    # and it is a different function: the plain recurrence misses by O(1)
    assert rel(oracle.ssd_fwd(**pr).y, ref) > 1e-2


def test_input_dt_is_the_plain_recurrence_on_scaled_input():
    # the input term delta x (outer) B is the plain one with x replaced by
    # delta x; outputs and final states agree when the skip is left out, and
    # the skip adds D x (the raw x) on top
    rng = np.random.default_rng(19)
    pr = rand_problem(rng, gated=False, with_D=False)
    delta = oracle.step_size(pr["dt"], pr["dt_bias"])
    a = oracle.ssd_fwd(**pr, input_dt=True)
    b = oracle.ssd_fwd(**dict(pr, x=pr["x"] * delta[..., None]))
    assert rel(a.y, b.y) < 1e-13 and rel(a.final_states, b.final_states) < 1e-13
    D = rng.standard_normal(pr["x"].shape[2])
    c = oracle.ssd_fwd(**dict(pr, D=D), input_dt=True)
    np.testing.assert_allclose(c.y - a.y, D[None, None, :, None] * pr["x"], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- special cases

def test_zero_decay_is_prefix_sum():
    # A = 0: exp(0) = 1 and the state is a running sum; with N = 1, B = C = 1
    # the output is numpy's cumulative sum of x plus the skip.
    rng = np.random.default_rng(3)
    b, T, H, P = 2, 50, 3, 4
    x = rng.standard_normal((b, T, H, P))
    ones = np.ones((b, T, 1, 1))
    dt = rng.standard_normal((b, T, H))
    D = rng.standard_normal(H)
    r = oracle.ssd_fwd(x, ones, ones, dt, np.zeros(H), D=D)
    ref = np.cumsum(x, axis=1) + D[None, None, :, None] * x
    np.testing.assert_allclose(r.y, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r.final_states[:, :, :, 0], x.sum(axis=1), rtol=0, atol=1e-13)
    # with the step size on the input term the sum is of delta x
    ri = oracle.ssd_fwd(x, ones, ones, dt, np.zeros(H), D=D, input_dt=True)
    dx = plain_softplus(dt)[..., None] * x
    np.testing.assert_allclose(ri.y, np.cumsum(dx, axis=1) + D[None, None, :, None] * x,
                               rtol=0, atol=1e-13)


def test_zero_decay_general_BC():
    # A = 0: y_t = sum_{s<=t} (C_t . B_s) x_s, i.e. causal linear attention.
    rng = np.random.default_rng(4)
    b, T, H, P, N = 1, 30, 2, 3, 4
    x = rng.standard_normal((b, T, H, P))
    B = rng.standard_normal((b, T, 1, N))
    C = rng.standard_normal((b, T, 1, N))
    dt = rng.standard_normal((b, T, H))
    r = oracle.ssd_fwd(x, B, C, dt, np.zeros(H))
    scores = np.tril(C[0, :, 0] @ B[0, :, 0].T)            # (T, T)
    ref = np.einsum("ts,shp->thp", scores, x[0])
    assert rel(r.y[0], ref) < 1e-13


def test_strong_decay_is_memoryless():
    # A = -1e4 with u > 0 gives a < -6900, exp(a) == 0 in fp64: no memory.
    rng = np.random.default_rng(5)
    b, T, H, P, N, G = 1, 20, 4, 3, 5, 2
    x = rng.standard_normal((b, T, H, P))
    B = rng.standard_normal((b, T, G, N))
    C = rng.standard_normal((b, T, G, N))
    dt = rng.uniform(0.1, 2.0, (b, T, H))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((b, H, P, N))
    r = oracle.ssd_fwd(x, B, C, dt, np.full(H, -1e4), D=D, initial_states=h0)
    cb = np.einsum("btgn,btgn->btg", C, B)
    cbh = np.repeat(cb, H // G, axis=2)
    ref = (cbh + D[None, None, :])[..., None] * x
    np.testing.assert_allclose(r.y, ref, rtol=1e-14, atol=1e-14)


def test_single_token():
    # T = 1: y = exp(a0) C.h0[p,:] + (C.B) x + D x  (the state update comes first)
    rng = np.random.default_rng(6)
    H, P, N = 2, 3, 4
    x = rng.standard_normal((1, 1, H, P))
    B = rng.standard_normal((1, 1, 1, N))
    C = rng.standard_normal((1, 1, 1, N))
    dt = rng.standard_normal((1, 1, H))
    A = np.array([-0.7, -2.0])
    bias = np.array([0.3, -1.0])
    D = np.array([0.25, -1.5])
    h0 = rng.standard_normal((1, H, P, N))
    r = oracle.ssd_fwd(x, B, C, dt, A, dt_bias=bias, D=D, initial_states=h0)
    for h in range(H):
        a = np.logaddexp(0.0, dt[0, 0, h] + bias[h]) * A[h]
        ref = (np.exp(a) * (h0[0, h] @ C[0, 0, 0]) + np.dot(C[0, 0, 0], B[0, 0, 0]) * x[0, 0, h]
               + D[h] * x[0, 0, h])
        np.testing.assert_allclose(r.y[0, 0, h], ref, rtol=1e-14)
        refS = np.exp(a) * h0[0, h] + np.outer(x[0, 0, h], B[0, 0, 0])
        np.testing.assert_allclose(r.final_states[0, h], refS, rtol=1e-14)


def test_constant_step_is_geometric():
    # Clamping the step to [d, d] makes abar = exp(d A) constant: the decay from
    # s to t is abar^(t-s), a power, independent of dt.
    rng = np.random.default_rng(8)
    b, T, H, P, N = 1, 25, 2, 2, 3
    x = rng.standard_normal((b, T, H, P))
    B = rng.standard_normal((b, T, 1, N))
    C = rng.standard_normal((b, T, 1, N))
    dt = 5 * rng.standard_normal((b, T, H))
    A = np.array([-0.5, -3.0])
    d = 0.05
    r = oracle.ssd_fwd(x, B, C, dt, A, dt_limit=(d, d))
    for h in range(H):
        q = math.exp(d * A[h])
        W = np.array([[q ** (t - s) if s <= t else 0.0 for s in range(T)] for t in range(T)])
        scores = W * (C[0, :, 0] @ B[0, :, 0].T)
        np.testing.assert_allclose(r.y[0, :, h], scores @ x[0, :, h], rtol=1e-12, atol=1e-13)


def test_no_softplus_uses_raw_step():
    rng = np.random.default_rng(9)
    pr = rand_problem(rng, b=1, T=12, gated=False, with_D=False, h0=False)
    r = oracle.ssd_fwd(**pr, dt_softplus=False)
    # closed form with delta = dt + bias (no softplus)
    x, B, C, dt, A, bias = (pr[k] for k in ("x", "B", "C", "dt", "A", "dt_bias"))
    H, G = x.shape[2], B.shape[2]
    for h in range(H):
        g = h // (H // G)
        abar = np.exp((dt[0, :, h] + bias[h]) * A[h])
        T = x.shape[1]
        for t in range(T):
            ref = sum(np.prod(abar[s + 1:t + 1]) * np.dot(C[0, t, g], B[0, s, g]) * x[0, s, h]
                      for s in range(t + 1))
            np.testing.assert_allclose(r.y[0, t, h], ref, rtol=1e-11, atol=1e-12)


def test_softplus_matches_library_and_threshold_form():
    u = np.concatenate([np.linspace(-40, 40, 4001), [-700.0, 700.0, 0.0]])
    np.testing.assert_allclose(oracle.softplus(u), np.logaddexp(0.0, u), rtol=1e-15, atol=0)
    # The GPU computes softplus(u) = u for u > 20; that differs from the exact
    # value by log1p(exp(-u)) <= 2.1e-9 relative.
    big = u[u > 20]
    assert np.max(np.abs(oracle.softplus(big) - big) / big) < 2.1e-9 + 1e-16


# ---------------------------------------------------------------- invariants

def test_split_resume_bit_exact():
    rng = np.random.default_rng(12)
    pr = rand_problem(rng, b=2, T=37)
    full = oracle.ssd_fwd(**pr)
    k = 15
    cut = lambda a, sl: None if a is None else a[:, sl]
    first = oracle.ssd_fwd(**{**pr, **{n: cut(pr[n], slice(0, k)) for n in ("x", "B", "C", "dt", "z")}})
    second = oracle.ssd_fwd(**{**pr, **{n: cut(pr[n], slice(k, None)) for n in ("x", "B", "C", "dt", "z")},
                               "initial_states": first.final_states})
    assert np.array_equal(np.concatenate([first.y, second.y], axis=1), full.y)
    assert np.array_equal(second.final_states, full.final_states)


def test_packed_equals_independent_runs_bit_exact():
    rng = np.random.default_rng(13)
    lens = [5, 0, 17, 1, 9]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    H, P, N, G = 4, 3, 2, 2
    x = rng.standard_normal((T, H, P)); B = rng.standard_normal((T, G, N))
    C = rng.standard_normal((T, G, N)); dt = rng.standard_normal((T, H))
    z = rng.standard_normal((T, H, P)); A = -np.exp(rng.uniform(0, 1, H))
    bias = rng.standard_normal(H); D = rng.standard_normal(H)
    h0 = rng.standard_normal((len(lens), H, P, N))
    packed = oracle.ssd_fwd(x, B, C, dt, A, bias, D, z, h0, cu_seqlens=cu)
    for i, L in enumerate(lens):
        s = cu[i]
        one = oracle.ssd_fwd(x[None, s:s + L], B[None, s:s + L], C[None, s:s + L],
                             dt[None, s:s + L], A, bias, D, z[None, s:s + L], h0[i:i + 1])
        assert np.array_equal(packed.y[s:s + L], one.y[0])
        assert np.array_equal(packed.final_states[i], one.final_states[0])
    # an empty sequence hands its initial state straight through
    assert np.array_equal(packed.final_states[1], h0[1])


def test_group_expansion_bit_exact():
    # G groups shared by H/G heads == H groups with each head's B, C repeated.
    rng = np.random.default_rng(14)
    pr = rand_problem(rng, b=1, T=19, H=6, G=2)
    grouped = oracle.ssd_fwd(**pr)
    rep = lambda a: np.repeat(a, 3, axis=2)
    expanded = oracle.ssd_fwd(**{**pr, "B": rep(pr["B"]), "C": rep(pr["C"])})
    assert np.array_equal(grouped.y, expanded.y)
    # and the mapping is contiguous: head 2 (group 0) differs from head 3 (group 1)
    swapped = oracle.ssd_fwd(**{**pr, "B": pr["B"][:, :, ::-1].copy()})
    assert not np.allclose(swapped.y[:, :, 0], grouped.y[:, :, 0])


def test_linearity_and_causality():
    rng = np.random.default_rng(15)
    pr = rand_problem(rng, b=1, T=21, gated=False)
    base = oracle.ssd_fwd(**pr).y
    # linear in (x, h0) jointly with the skip: scale both by 3
    s = oracle.ssd_fwd(**{**pr, "x": 3 * pr["x"], "initial_states": 3 * pr["initial_states"]}).y
    np.testing.assert_allclose(s, 3 * base, rtol=1e-13, atol=1e-13)
    # linear in C (the skip does not depend on C): y(C1 + C2) = y(C1) + y(C2) - D x
    C2 = rng.standard_normal(pr["C"].shape)
    y12 = oracle.ssd_fwd(**{**pr, "C": pr["C"] + C2}).y
    y2 = oracle.ssd_fwd(**{**pr, "C": C2}).y
    Dx = pr["D"][None, None, :, None] * pr["x"]
    np.testing.assert_allclose(y12, base + y2 - Dx, rtol=1e-12, atol=1e-12)
    # causality: change token 10 only, outputs before it are unchanged
    x2 = pr["x"].copy(); x2[:, 10] += 1.0
    dt2 = pr["dt"].copy(); dt2[:, 10] -= 2.0
    y3 = oracle.ssd_fwd(**{**pr, "x": x2, "dt": dt2}).y
    assert np.array_equal(y3[:, :10], base[:, :10])
    assert not np.allclose(y3[:, 10:], base[:, 10:])
    # B = 0 and no initial state: only the skip remains
    yb = oracle.ssd_fwd(**{**pr, "B": np.zeros_like(pr["B"]), "initial_states": None}).y
    np.testing.assert_allclose(yb, Dx, rtol=0, atol=0)
    # z = 0 gates everything off
    yz = oracle.ssd_fwd(**{**pr, "z": np.zeros_like(pr["x"])}).y
    assert np.all(yz == 0.0)


# ---------------------------------------------------------------- chunkwise decomposition

def chunkwise_eval(x, B, C, dt, A, dt_bias, D, z, h0, Cs, window_shift=1):
    """A chunked evaluation of the recurrence, worked out from it chunk by chunk.

    For one batch row, real A, groups mapped to heads as g = h // (H/G).  The
    token axis is cut into chunks of Cs tokens (the last one shorter).  Inside
    chunk c with local positions 0..L-1 and per-head log-decays a_t:
      * cs[l] = a_0 + ... + a_l, the chunk's cumulative log-decay (SSD
        Reference, "Chunking and the discretized log-decay");
      * the intra-chunk output y_l += sum_{s<=l} exp(cs[l] - cs[s]) (C_l.B_s) x_s,
        and the chunk's end state from a zero start
        S_c = sum_s exp(cs[L-1] - cs[s]) x_s (outer) B_s ("Intra-chunk outputs
        and per-chunk states"); the exponent is selected before it is taken,
        so masked pairs never reach exp;
      * the state entering chunk z is the sum over earlier chunks c of
        exp(CD[z-1] - CD[c]) S_c plus exp(CD[z-1]) h0, CD being the running
        sum of the chunks' total log-decays and CD[-1] = 0 ("Inter-chunk
        propagation", the decay_chunk window); ``window_shift=0`` evaluates
        the off-by-one window CD[z] - CD[c] the page warns about instead;
      * the readout y_l += exp(cs[l]) C_l . Hin_z ("Readout").
    The skip D x and the gate silu(z) are applied last.  Returns
    (y, final state, chunk end states, carry-in states).
    """
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    hpg = H // G
    starts = list(range(0, T, Cs))
    nc = len(starts)
    a = plain_softplus(dt + dt_bias[None]) * A[None]          # (T, H)
    y = np.zeros((T, H, P))
    S = np.zeros((nc, H, P, N))
    lam = np.zeros((nc, H))
    css = []
    for c, t0 in enumerate(starts):
        L = min(Cs, T - t0)
        cs = np.zeros((L, H))
        run = np.zeros(H)
        for l in range(L):
            run = run + a[t0 + l]
            cs[l] = run
        css.append(cs)
        lam[c] = cs[L - 1]
        for h in range(H):
            g = h // hpg
            Cg, Bg, xh = C[t0:t0 + L, g], B[t0:t0 + L, g], x[t0:t0 + L, h]
            for l in range(L):
                for s_ in range(l + 1):
                    y[t0 + l, h] += np.exp(cs[l, h] - cs[s_, h]) * np.dot(Cg[l], Bg[s_]) * xh[s_]
            for s_ in range(L):
                S[c, h] += np.exp(cs[L - 1, h] - cs[s_, h]) * np.outer(xh[s_], Bg[s_])
    CD = np.cumsum(lam, axis=0)                               # (nc, H)
    Hin = np.zeros((nc, H, P, N))
    for zc in range(nc):
        top = CD[zc - 1] if (window_shift and zc > 0) else (np.zeros(H) if window_shift else CD[zc])
        for c in range(zc):
            Hin[zc] += np.exp(top - CD[c])[:, None, None] * S[c]
        if h0 is not None:
            Hin[zc] += np.exp(top)[:, None, None] * h0
    for c, t0 in enumerate(starts):
        cs = css[c]
        for l in range(cs.shape[0]):
            for h in range(H):
                y[t0 + l, h] += np.exp(cs[l, h]) * (Hin[c, h] @ C[t0 + l, h // hpg])
    if D is not None:
        y = y + D[None, :, None] * x
    if z is not None:
        y = y * z / (1.0 + np.exp(-z))
    final = np.exp(lam[-1])[:, None, None] * Hin[-1] + S[-1]
    return y, final, S, Hin


@pytest.mark.parametrize("T,Cs", [(64, 16), (61, 16), (16, 16), (5, 16), (47, 8)])
def test_oracle_matches_chunkwise_evaluation(T, Cs):
    rng = np.random.default_rng(20 + T)
    H, P, N, G = 4, 3, 5, 2
    x = rng.standard_normal((T, H, P)); B = rng.standard_normal((T, G, N))
    C = rng.standard_normal((T, G, N)); dt = rng.standard_normal((T, H))
    z = rng.standard_normal((T, H, P)); A = -np.exp(rng.uniform(-2, 1.5, H))
    bias = rng.uniform(-3, 0, H); D = rng.standard_normal(H)
    h0 = rng.standard_normal((1, H, P, N))
    r = oracle.ssd_fwd(x[None], B[None], C[None], dt[None], A, bias, D, z[None], h0,
                       chunk_size=Cs)
    Y, final, states, carry = chunkwise_eval(x, B, C, dt, A, bias, D, z, h0[0], Cs)
    assert rel(r.y[0], Y) < 1e-12
    assert rel(r.final_states[0], final) < 1e-12
    # the oracle's stage helpers agree with the pages' per-chunk quantities
    meta = oracle.batch_chunk_meta(1, T, Cs)
    S = oracle.chunk_states(x, B, dt, A, meta, dt_bias=bias)
    assert rel(S, states) < 1e-12
    Hin = oracle.carry_in_states(r.chunk_end_states, meta, h0)
    assert rel(Hin, carry) < 1e-12
    # the chunk-level recurrence on the isolated chunk states lands on the same
    # carry-in and final states as the token-level recurrence
    Hin2, fin2 = oracle.state_passing(S, oracle.chunk_cumsum(dt, A, meta, Cs, dt_bias=bias),
                                      meta, h0)
    assert rel(Hin2, carry) < 1e-12
    assert rel(fin2[0], final) < 1e-12
    cs = oracle.chunk_cumsum(dt, A, meta, Cs, dt_bias=bias)
    a = plain_softplus(dt + bias) * A
    for j in range(meta.nchunks):
        s0, L = meta.start[j], meta.length[j]
        np.testing.assert_allclose(cs[j, :, :L].T, np.cumsum(a[s0:s0 + L], 0), rtol=1e-13, atol=1e-13)
        assert np.all(cs[j, :, L:] == cs[j, :, L - 1:L])   # flat past a short chunk's end
    CB = oracle.bmm_chunk(C, B, meta, Cs)
    for j in range(meta.nchunks):
        s0, L = meta.start[j], meta.length[j]
        for g in range(G):
            ref = np.array([[np.dot(C[s0 + l, g], B[s0 + s, g]) for s in range(L)] for l in range(L)])
            np.testing.assert_allclose(CB[j, g, :L, :L], ref, rtol=1e-14, atol=1e-14)


def test_wrong_propagation_window_is_detected():
    # Time-varying dt distinguishes the correct window CD[z-1] - CD[c] from the
    # off-by-one CD[z] - CD[c] (SSD Reference, "Inter-chunk propagation",
    # correctness note).  Guard that the decomposition test would catch it.
    rng = np.random.default_rng(31)
    T, Cs, H, P, N = 48, 8, 2, 2, 3
    x = rng.standard_normal((T, H, P)); B = rng.standard_normal((T, 1, N))
    C = rng.standard_normal((T, 1, N)); dt = rng.standard_normal((T, H))
    A = -np.exp(rng.uniform(-1, 1, H)); bias = np.zeros(H)
    r = oracle.ssd_fwd(x[None], B[None], C[None], dt[None], A, bias)
    meta = oracle.batch_chunk_meta(1, T, Cs)
    S = oracle.chunk_states(x, B, dt, A, meta, dt_bias=bias)
    cs = oracle.chunk_cumsum(dt, A, meta, Cs, dt_bias=bias)
    Lam = cs[:, :, -1]
    CD = np.cumsum(Lam, 0)
    nc = meta.nchunks
    wrong = np.zeros_like(S)
    for zc in range(nc):
        for c in range(zc):
            wrong[zc] += np.exp(CD[zc] - CD[c])[:, None, None] * S[c]
    Hin = oracle.carry_in_states(oracle.ssd_fwd(x[None], B[None], C[None], dt[None], A, bias,
                                                chunk_size=Cs).chunk_end_states, meta)
    assert rel(wrong, Hin) > 1e-3
    # the chunked evaluation with that window is a different function, and
    # the oracle is not it (while the correct window matches, above)
    yw = chunkwise_eval(x, B, C, dt, A, bias, None, None, None, Cs, window_shift=0)[0]
    assert rel(yw, r.y[0]) > 1e-3
    yr = chunkwise_eval(x, B, C, dt, A, bias, None, None, None, Cs)[0]
    assert rel(yr, r.y[0]) < 1e-12


def test_state_passing_packed_with_empty_sequence():
    rng = np.random.default_rng(41)
    lens = [7, 0, 12, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, H, P, N, Cs = int(cu[-1]), 2, 2, 3, 4
    x = rng.standard_normal((T, H, P)); B = rng.standard_normal((T, 1, N))
    C = rng.standard_normal((T, 1, N)); dt = rng.standard_normal((T, H))
    A = -np.exp(rng.uniform(-1, 1, H)); h0 = rng.standard_normal((4, H, P, N))
    r = oracle.ssd_fwd(x, B, C, dt, A, initial_states=h0, cu_seqlens=cu, chunk_size=Cs)
    meta = oracle.varlen_chunk_meta(cu, Cs)
    S = oracle.chunk_states(x, B, dt, A, meta)
    cs = oracle.chunk_cumsum(dt, A, meta, Cs)
    Hin, fin = oracle.state_passing(S, cs, meta, h0)
    assert rel(Hin, oracle.carry_in_states(r.chunk_end_states, meta, h0)) < 1e-12
    assert rel(fin, r.final_states) < 1e-12
    assert np.array_equal(fin[1], h0[1])


# ---------------------------------------------------------------- the step-size clamp (numpy helpers)

def test_numpy_clamp_pinned_to_constant_step_and_to_the_c_oracle():
    # oracle.step_size / oracle.chunk_cumsum (numpy) are the references of the
    # GPU's chunk cumsum; their clamp is tied here to a closed form and to the
    # C oracle's clamp.
    rng = np.random.default_rng(51)
    T, H, Cs = 45, 3, 16
    dt = rng.standard_normal((T, H)) * 3.0
    bias = rng.uniform(-2, 1, H)
    A = -np.exp(rng.uniform(-1, 1, H))
    meta = oracle.batch_chunk_meta(1, T, Cs)
    # a degenerate limit [d, d] makes every step d: the cumsum is l * d * A
    d = 0.0375
    cs = oracle.chunk_cumsum(dt, A, meta, Cs, dt_bias=bias, dt_limit=(d, d))
    for j in range(meta.nchunks):
        L = meta.length[j]
        ref = np.outer(A, np.arange(1, Cs + 1).clip(max=L)) * d
        np.testing.assert_allclose(cs[j], ref, rtol=1e-13, atol=0)
    # the clamp bounds the softplus value from both sides and leaves the rest
    lo, hi = 0.3, 1.1
    sp = plain_softplus(dt + bias)
    st = oracle.step_size(dt, bias, dt_limit=(lo, hi))
    assert np.max(np.abs(st - np.clip(sp, lo, hi))) < 1e-15
    assert np.any(sp < lo) and np.any(sp > hi) and np.any((sp > lo) & (sp < hi))
    # the C oracle with its clamp equals the C oracle fed the numpy steps
    # directly (no softplus, no bias)
    P, N = 2, 3
    x = rng.standard_normal((1, T, H, P)); B = rng.standard_normal((1, T, 1, N))
    C = rng.standard_normal((1, T, 1, N))
    rc = oracle.ssd_fwd(x, B, C, dt[None], A, dt_bias=bias, dt_limit=(lo, hi))
    rn = oracle.ssd_fwd(x, B, C, st[None], A, dt_softplus=False)
    assert rel(rc.y, rn.y) < 1e-13
    assert rel(rc.final_states, rn.final_states) < 1e-13
