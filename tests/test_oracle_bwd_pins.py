"""Pins of the oracle's backward (``oracle.ssd_bwd``) against things other than itself.

* Central finite differences of the forward oracle, in fp64, along random
  directions of every input (the check cudnn-frontend PR 1133 describes: all
  gradients against fp64 references), on small problems that cover groups, the
  gate, the skip, initial and final states, packed sequences with empty ones,
  softplus off and the clamp.
* Exact adjoint identities: the loss is affine in x, C, D and the initial
  state and (for a zero initial state) linear in B, so a finite step of any
  size must change it by exactly <gradient, step> (up to rounding).
* A closed form: with A = 0, N = 1 and B = C = 1 the output is a prefix sum, so
  dx is the reverse cumulative sum of dout plus D dout (with the step size on
  the input term, delta times it, and the raw dt gets x . that sum through
  softplus').
* The same checks with the step size on the input term (``input_dt``).
* Structure: grouped B/C gradients equal the per-head gradients summed over
  the group, and a packed batch equals its sequences run one by one.
"""
import numpy as np
import pytest

import oracle


def problem(seed, b=2, T=9, H=4, P=3, G=2, N=2, z=True, D=True, h0=True, dfinal=True,
            cu=None):
    rng = np.random.default_rng(seed)
    lead = (cu[-1],) if cu is not None else (b, T)
    nseq = len(cu) - 1 if cu is not None else b
    p = dict(
        x=rng.standard_normal(lead + (H, P)),
        B=rng.standard_normal(lead + (G, N)),
        C=rng.standard_normal(lead + (G, N)),
        dt=rng.standard_normal(lead + (H,)),
        A=-np.exp(rng.uniform(np.log(0.5), np.log(4.0), H)),
        dt_bias=rng.uniform(-2.0, 0.5, H),
        D=rng.standard_normal(H) if D else None,
        z=rng.standard_normal(lead + (H, P)) if z else None,
        initial_states=rng.standard_normal((nseq, H, P, N)) if h0 else None,
    )
    w = dict(dout=rng.standard_normal(lead + (H, P)),
             dfinal=rng.standard_normal((nseq, H, P, N)) if dfinal else None)
    return p, w, cu


def loss(p, w, cu, **kw):
    r = oracle.ssd_fwd(p["x"], p["B"], p["C"], p["dt"], p["A"], dt_bias=p["dt_bias"], D=p["D"],
                       z=p["z"], initial_states=p["initial_states"], cu_seqlens=cu, **kw)
    L = float(np.sum(w["dout"] * r.y))
    if w["dfinal"] is not None:
        L += float(np.sum(w["dfinal"] * r.final_states))
    return L


def grads(p, w, cu, **kw):
    return oracle.ssd_bwd(p["x"], p["B"], p["C"], p["dt"], p["A"], w["dout"],
                          dt_bias=p["dt_bias"], D=p["D"], z=p["z"],
                          initial_states=p["initial_states"], dfinal_states=w["dfinal"],
                          cu_seqlens=cu, **kw)


GRAD_OF = {"x": "dx", "B": "dB", "C": "dC", "dt": "ddt", "A": "dA", "dt_bias": "ddt_bias",
           "D": "dD", "z": "dz", "initial_states": "dinitial_states"}


def check_fd(p, w, cu, eps=1e-6, ndir=3, rtol=2e-7, seed=7, **kw):
    g = grads(p, w, cu, **kw)
    rng = np.random.default_rng(seed)
    for name, gname in GRAD_OF.items():
        if p[name] is None:
            continue
        for _ in range(ndir):
            v = rng.standard_normal(np.shape(p[name]))
            hi = dict(p); hi[name] = p[name] + eps * v
            lo = dict(p); lo[name] = p[name] - eps * v
            fd = (loss(hi, w, cu, **kw) - loss(lo, w, cu, **kw)) / (2 * eps)
            an = float(np.sum(getattr(g, gname) * v))
            scale = max(1.0, abs(fd))
            assert abs(fd - an) <= rtol * scale, f"{name}: fd {fd:.12g} vs grad {an:.12g}"


def test_fd_batch_all_options():
    check_fd(*problem(1))


def test_fd_packed_with_empty_sequences():
    cu = np.array([0, 4, 4, 5, 11, 11], dtype=np.int64)
    check_fd(*problem(2, cu=cu))


def test_fd_no_gate_no_skip_no_states():
    check_fd(*problem(3, z=False, D=False, h0=False, dfinal=False))


def test_fd_heads_per_group_odd():
    check_fd(*problem(4, H=6, G=2, P=2, N=3))


def test_fd_without_softplus():
    p, w, cu = problem(5)
    p["dt"] = np.abs(p["dt"]) * 0.3 + 0.05
    p["dt_bias"] = np.zeros_like(p["dt_bias"])
    check_fd(p, w, cu, dt_softplus=False)


@pytest.mark.parametrize("kw", [dict(), dict(cu=np.array([0, 4, 4, 5, 11, 11], dtype=np.int64)),
                                dict(z=False, D=False, h0=False, dfinal=False)],
                         ids=["batch", "packed", "plain"])
def test_fd_input_dt(kw):
    check_fd(*problem(13, **kw), input_dt=True)


def test_fd_input_dt_clamp_and_no_softplus():
    p, w, cu = problem(14, T=12)
    delta = oracle.step_size(p["dt"], p["dt_bias"])
    lo, hi = np.quantile(delta, [0.25, 0.75])
    for v in (lo, hi):
        assert not (np.abs(delta - v) < 1e-4).any()
    g = grads(p, w, cu, dt_limit=(lo, hi), input_dt=True)
    assert np.all(g.ddt[(delta < lo) | (delta > hi)] == 0.0)
    check_fd(p, w, cu, dt_limit=(lo, hi), input_dt=True)
    q, w2, cu2 = problem(15)
    q["dt"] = np.abs(q["dt"]) * 0.3 + 0.05
    q["dt_bias"] = np.zeros_like(q["dt_bias"])
    check_fd(q, w2, cu2, dt_softplus=False, input_dt=True)


def test_fd_clamp_active():
    p, w, cu = problem(6, T=12)
    delta = oracle.step_size(p["dt"], p["dt_bias"])
    lo, hi = np.quantile(delta, [0.25, 0.75])
    # keep every step away from the clamp edges by more than the FD step
    for v in (lo, hi):
        near = np.abs(delta - v) < 1e-4
        assert not near.any()
    g = grads(p, w, cu, dt_limit=(lo, hi))
    clamped = (delta < lo) | (delta > hi)
    assert clamped.any() and (~clamped).any()
    assert np.all(g.ddt[clamped] == 0.0)
    check_fd(p, w, cu, dt_limit=(lo, hi))


@pytest.mark.parametrize("name", ["x", "C", "D", "initial_states", "B"])
def test_affine_identity_exact(name):
    # zero initial state for B (the loss is linear in B only then)
    p, w, cu = problem(8, h0=(name != "B"))
    g = grads(p, w, cu)
    rng = np.random.default_rng(9)
    v = rng.standard_normal(np.shape(p[name]))
    q = dict(p); q[name] = p[name] + v
    if name == "B":
        # L(B) is linear in B only with x fixed and a zero initial state: the
        # gradient at B = 0 is exact for any step
        p0 = dict(p); p0["B"] = np.zeros_like(p["B"])
        g0 = grads(p0, w, cu)
        dL = loss(dict(p0, B=v), w, cu) - loss(p0, w, cu)
        an = float(np.sum(g0.dB * v))
    else:
        dL = loss(q, w, cu) - loss(p, w, cu)
        an = float(np.sum(getattr(g, GRAD_OF[name]) * v))
    assert abs(dL - an) <= 1e-11 * max(1.0, abs(dL))


def test_prefix_sum_closed_form():
    rng = np.random.default_rng(10)
    T, H, P = 13, 2, 3
    x = rng.standard_normal((1, T, H, P))
    ones = np.ones((1, T, 1, 1))
    dt = rng.standard_normal((1, T, H))
    D = rng.standard_normal(H)
    dout = rng.standard_normal((1, T, H, P))
    g = oracle.ssd_bwd(x, ones, ones, dt, np.zeros(H), dout, D=D)
    rev = np.cumsum(dout[:, ::-1], axis=1)[:, ::-1]
    assert np.allclose(g.dx, rev + D[None, None, :, None] * dout, rtol=0, atol=1e-13)
    # A = 0: nothing depends on dt
    assert np.all(g.ddt == 0.0) and np.all(g.ddt_bias == 0.0)
    # with the step size on the input: y_t = sum_{s<=t} delta_s x_s + D x_t
    delta = np.log1p(np.exp(dt))
    gi = oracle.ssd_bwd(x, ones, ones, dt, np.zeros(H), dout, D=D, input_dt=True)
    assert np.allclose(gi.dx, delta[..., None] * rev + D[None, None, :, None] * dout,
                       rtol=0, atol=1e-13)
    sig = 1.0 / (1.0 + np.exp(-dt))
    assert np.allclose(gi.ddt, np.sum(x * rev, axis=-1) * sig, rtol=0, atol=1e-13)
    assert np.allclose(gi.ddt_bias, gi.ddt.sum(axis=(0, 1)), rtol=0, atol=1e-13)


def test_group_gradients_are_head_sums():
    p, w, cu = problem(11, H=4, G=2)
    g = grads(p, w, cu)
    # expand to one group per head: B and C repeated
    q = dict(p)
    q["B"] = np.repeat(p["B"], 2, axis=2)
    q["C"] = np.repeat(p["C"], 2, axis=2)
    e = grads(q, w, cu)
    for name in ("dB", "dC"):
        per_head = getattr(e, name)
        summed = per_head.reshape(per_head.shape[:2] + (2, 2, -1)).sum(axis=3)
        assert np.allclose(getattr(g, name), summed, rtol=1e-13, atol=1e-13)
    assert np.array_equal(g.dx, e.dx) and np.array_equal(g.ddt, e.ddt)


def test_packed_equals_sequences_one_by_one():
    cu = np.array([0, 3, 3, 10, 16], dtype=np.int64)
    p, w, _ = problem(12, cu=cu)
    g = grads(p, w, cu)
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        sub = {k: (v[a:b] if k in ("x", "B", "C", "dt", "z") else v) for k, v in p.items()}
        sub["initial_states"] = p["initial_states"][i:i + 1]
        ws = dict(dout=w["dout"][a:b], dfinal=w["dfinal"][i:i + 1])
        gi = grads(sub, ws, np.array([0, b - a], dtype=np.int64))
        assert np.array_equal(g.dx[a:b], gi.dx)
        assert np.array_equal(g.ddt[a:b], gi.ddt)
        assert np.array_equal(g.dz[a:b], gi.dz)
        assert np.array_equal(g.dinitial_states[i], gi.dinitial_states[0])
        # the group sums over heads are formed per token, so they match too
        assert np.array_equal(g.dB[a:b], gi.dB) and np.array_equal(g.dC[a:b], gi.dC)
