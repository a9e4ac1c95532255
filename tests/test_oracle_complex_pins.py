"""Pins of the complex-A oracle (``oracle.ssd_complex_fwd``) against facts other
than itself.

* With every imaginary part zero it is the real recurrence: the pinned real
  oracle (one group per head) gives the same output, and the imaginary part is
  exactly zero.
* Brute force of the closed form (SSD Reference, "Math": y_t = sum_{s<=t}
  C_t^T (prod_{u=s+1..t} abar_u) B_s x_s) with explicit products of per-token
  complex decays.
* A pure rotation (A = i w, N = D = 1, B = C = 1) has the closed form
  y_t = e^{i phi_t} sum_{s<=t} e^{-i phi_s} x_s with phi = w cumsum(delta).
* The recurrence is holomorphic in its inputs (no conjugation anywhere), so
  conjugating x, B, C and A conjugates y.
* A chunked evaluation worked out here chunk by chunk (SSD Reference: the
  within-chunk cumulative log-decay, the intra-chunk outputs and chunk end
  states, the inter-chunk window exp(CD[z-1] - CD[c]) with the init term
  exp(CD[z-1]) H_{-1}, the readout) agrees with it for time-varying dt, a
  ragged last chunk and an initial state in the (D, N) layout.
* Split and resume, and packed sequences run one by one, agree bit for bit.
"""
import numpy as np
import pytest

import oracle


def cnormal(rng, shape):
    return rng.standard_normal(shape) + 1j * rng.standard_normal(shape)


def problem(seed, b=2, T=11, H=3, D=4, N=5, h0=False):
    rng = np.random.default_rng(seed)
    x = cnormal(rng, (b, T, H, D))
    B = cnormal(rng, (b, T, H, N))
    C = cnormal(rng, (b, T, H, N))
    dt = rng.standard_normal((b, T, H))
    A = -np.exp(rng.uniform(np.log(0.3), np.log(2.0), H)) + 1j * rng.uniform(-3.0, 3.0, H)
    init = cnormal(rng, (b, H, D, N)) if h0 else None
    return x, B, C, dt, A, init


def softplus(u):
    return np.log1p(np.exp(u))


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_real_case_is_the_real_recurrence():
    rng = np.random.default_rng(1)
    b, T, H, D, N = 2, 17, 3, 4, 5
    x = rng.standard_normal((b, T, H, D))
    B = rng.standard_normal((b, T, H, N))
    C = rng.standard_normal((b, T, H, N))
    dt = rng.standard_normal((b, T, H))
    A = -np.exp(rng.uniform(0.0, 1.0, H))
    h0 = rng.standard_normal((b, H, D, N))
    rc = oracle.ssd_complex_fwd(x, B, C, dt, A, initial_states=h0)
    rr = oracle.ssd_fwd(x, B, C, dt, A, initial_states=h0)  # one group per head
    assert np.all(rc.y.imag == 0.0) and np.all(rc.final_states.imag == 0.0)
    assert rel(rc.y.real, rr.y) < 1e-13
    assert rel(rc.final_states.real, rr.final_states) < 1e-13


def closed_form(x, B, C, dt, A):
    b, T, H, D = x.shape
    y = np.zeros_like(x, dtype=np.complex128)
    for bi in range(b):
        for h in range(H):
            abar = np.exp(softplus(dt[bi, :, h]) * A[h])
            for t in range(T):
                acc = np.zeros(D, dtype=np.complex128)
                for s in range(t + 1):
                    w = np.prod(abar[s + 1:t + 1])  # empty product is 1
                    acc += w * np.sum(C[bi, t, h] * B[bi, s, h]) * x[bi, s, h]
                y[bi, t, h] = acc
    return y


def test_closed_form_brute_force():
    x, B, C, dt, A, _ = problem(2)
    r = oracle.ssd_complex_fwd(x, B, C, dt, A)
    assert rel(r.y, closed_form(x, B, C, dt, A)) < 1e-12


def test_pure_rotation():
    rng = np.random.default_rng(3)
    T = 40
    x = cnormal(rng, (1, T, 1, 1))
    ones = np.ones((1, T, 1, 1), dtype=complex)
    dt = rng.standard_normal((1, T, 1))
    w = 1.7
    r = oracle.ssd_complex_fwd(x, ones, ones, dt, np.array([1j * w]))
    phi = w * np.cumsum(softplus(dt[0, :, 0]))
    ref = np.exp(1j * phi) * np.cumsum(np.exp(-1j * phi) * x[0, :, 0, 0])
    assert rel(r.y[0, :, 0, 0], ref) < 1e-12
    # no decay: the state's magnitude is the magnitude of the rotated sum
    assert np.allclose(np.abs(r.final_states[0, 0, 0, 0]), np.abs(ref[-1]), rtol=1e-12)


def test_conjugation_symmetry():
    x, B, C, dt, A, h0 = problem(4, h0=True)
    a = oracle.ssd_complex_fwd(x, B, C, dt, A, initial_states=h0)
    c = oracle.ssd_complex_fwd(x.conj(), B.conj(), C.conj(), dt, A.conj(),
                               initial_states=h0.conj())
    assert rel(c.y, a.y.conj()) < 1e-14
    assert rel(c.final_states, a.final_states.conj()) < 1e-14


def chunkwise_eval(x, B, C, dt, A, chunk, initial_states=None, window_shift=1):
    """A chunked evaluation of the complex recurrence, chunk by chunk.

    x (b, T, H, D), B and C (b, T, H, N) complex, dt (b, T, H) real, A (H)
    complex.  Each chunk of ``chunk`` tokens (the last one shorter) with
    per-token complex log-decays a_t = softplus(dt_t) A_h:
      * cs[l] = a_0 + ... + a_l (SSD Reference, "Chunking and the discretized
        log-decay");
      * intra-chunk output y_l = sum_{s<=l} exp(cs[l] - cs[s]) (C_l . B_s) x_s
        and the end state from zero S = sum_s exp(cs[L-1] - cs[s]) x_s (outer) B_s
        in the (D, N) layout ("Intra-chunk outputs and per-chunk states");
      * the state entering chunk z, sum_{c<z} exp(CD[z-1] - CD[c]) S_c plus
        exp(CD[z-1]) H_-1, CD the running sum of the chunks' total log-decays,
        CD[-1] = 0 ("Inter-chunk propagation"); ``window_shift=0`` uses the
        off-by-one window CD[z] - CD[c] instead;
      * the readout y_l += exp(cs[l]) sum_n C_l[n] Hin[:, n] ("Readout").
    Nothing is conjugated.  Returns y (b, T, H, D) complex.
    """
    b, T, H, Dm = x.shape
    N = B.shape[-1]
    starts = list(range(0, T, chunk))
    nc = len(starts)
    y = np.zeros((b, T, H, Dm), dtype=np.complex128)
    for bi in range(b):
        a = softplus(dt[bi]) * A[None, :]                        # (T, H) complex
        S = np.zeros((nc, H, Dm, N), dtype=np.complex128)
        lam = np.zeros((nc, H), dtype=np.complex128)
        css = []
        for c, t0 in enumerate(starts):
            L = min(chunk, T - t0)
            cs = np.cumsum(a[t0:t0 + L], axis=0)
            css.append(cs)
            lam[c] = cs[L - 1]
            for h in range(H):
                xh, Bh, Ch = x[bi, t0:t0 + L, h], B[bi, t0:t0 + L, h], C[bi, t0:t0 + L, h]
                for l in range(L):
                    for s_ in range(l + 1):
                        y[bi, t0 + l, h] += (np.exp(cs[l, h] - cs[s_, h])
                                             * np.sum(Ch[l] * Bh[s_]) * xh[s_])
                for s_ in range(L):
                    S[c, h] += np.exp(cs[L - 1, h] - cs[s_, h]) * np.outer(xh[s_], Bh[s_])
        CD = np.cumsum(lam, axis=0)
        for zc in range(nc):
            if window_shift:
                top = CD[zc - 1] if zc > 0 else np.zeros(H, dtype=np.complex128)
            else:
                top = CD[zc]
            Hin = np.zeros((H, Dm, N), dtype=np.complex128)
            for c in range(zc):
                Hin += np.exp(top - CD[c])[:, None, None] * S[c]
            if initial_states is not None:
                Hin += np.exp(top)[:, None, None] * initial_states[bi]
            t0 = starts[zc]
            cs = css[zc]
            for l in range(cs.shape[0]):
                for h in range(H):
                    y[bi, t0 + l, h] += np.exp(cs[l, h]) * (Hin[h] @ C[bi, t0 + l, h])
    return y


@pytest.mark.parametrize("T,chunk", [(16, 4), (23, 4), (20, 8), (5, 8)])
def test_matches_chunkwise_evaluation(T, chunk):
    x, B, C, dt, A, h0 = problem(5, T=T, h0=True)
    r = oracle.ssd_complex_fwd(x, B, C, dt, A, initial_states=h0)
    ref = chunkwise_eval(x, B, C, dt, A, chunk, initial_states=h0)
    assert rel(r.y, ref) < 1e-11
    assert rel(r.y.real, ref.real) < 1e-11


def test_propagation_window_matters():
    # the off-by-one the page warns about (CD[z] instead of CD[z-1]) is a
    # different function for time-varying dt, and the oracle is not it
    x, B, C, dt, A, _ = problem(6, T=16)
    r = oracle.ssd_complex_fwd(x, B, C, dt, A)
    assert rel(r.y, chunkwise_eval(x, B, C, dt, A, 4)) < 1e-11
    wrong = chunkwise_eval(x, B, C, dt, A, 4, window_shift=0)
    assert rel(wrong, r.y) > 1e-3


def test_split_resume_and_packed_bit_exact():
    x, B, C, dt, A, h0 = problem(7, T=19, h0=True)
    full = oracle.ssd_complex_fwd(x, B, C, dt, A, initial_states=h0)
    a = oracle.ssd_complex_fwd(x[:, :8], B[:, :8], C[:, :8], dt[:, :8], A, initial_states=h0)
    c = oracle.ssd_complex_fwd(x[:, 8:], B[:, 8:], C[:, 8:], dt[:, 8:], A,
                               initial_states=a.final_states)
    assert np.array_equal(np.concatenate([a.y, c.y], 1), full.y)
    assert np.array_equal(c.final_states, full.final_states)
    # two batch rows packed as sequences equal the batch run
    cu = np.array([0, 19, 38], dtype=np.int64)
    pk = oracle.ssd_complex_fwd(x.reshape(38, *x.shape[2:]), B.reshape(38, *B.shape[2:]),
                                C.reshape(38, *C.shape[2:]), dt.reshape(38, -1), A,
                                initial_states=h0, cu_seqlens=cu)
    assert np.array_equal(pk.y.reshape(full.y.shape), full.y)
