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
* The pages' own chunkwise algorithm (SSD Reference: padding rule, A_cumsum,
  L = exp(segsum) masked, Y_diag, states, decay_chunk[z, c] =
  exp(CD[z-1] - CD[c]) 1[z > c], the init term exp(CD[z-1]) H_{-1}, Y_off),
  written out here with numpy, agrees with it for time-varying dt, a ragged
  last chunk and an initial state in the (D, N) layout.
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


def pages_chunkwise(x, B, C, dt, A, chunk, initial_states=None, window_off_by_one=False):
    """The chunkwise evaluation the SSD Reference page describes, in numpy."""
    b, T, H, D = x.shape
    N = B.shape[-1]
    pad = (chunk - T % chunk) % chunk
    padt = lambda a: np.concatenate([a, np.zeros((b, pad) + a.shape[2:], dtype=a.dtype)], 1)
    x, B, C, dt = padt(x), padt(B), padt(C), padt(dt)
    nc = (T + pad) // chunk
    A_log = softplus(dt) * A[None, None, :]
    ch = lambda a: a.reshape((b, nc, chunk) + a.shape[2:])
    Xc, Bc, Cc, Ac = ch(x), ch(B), ch(C), ch(A_log)
    A_cumsum = np.cumsum(Ac, axis=2)                                   # (b, c, l, h)
    decay_states = np.exp(A_cumsum[:, :, -1:, :] - A_cumsum)
    seg = A_cumsum[:, :, :, None, :] - A_cumsum[:, :, None, :, :]     # (b, c, l, s, h)
    mask = np.tril(np.ones((chunk, chunk), dtype=bool))[None, None, :, :, None]
    L = np.where(mask, np.exp(np.where(mask, seg, 0.0)), 0.0)
    Y_diag = np.einsum("bclhn,bcshn,bclsh,bcshp->bclhp", Cc, Bc, L, Xc)
    states = np.einsum("bclhn,bclh,bclhp->bchpn", Bc, decay_states, Xc)  # (b, c, h, D, N)
    lam = A_cumsum[:, :, -1, :]                                        # (b, c, h)
    CD = np.cumsum(lam, axis=1)
    CDm1 = np.concatenate([np.zeros_like(CD[:, :1]), CD[:, :-1]], 1)   # CD[z-1], CD[-1] = 0
    Gz = np.zeros((b, nc, H, D, N), dtype=np.complex128)
    for z in range(nc):
        for c in range(z):
            top = CD[:, z] if window_off_by_one else CDm1[:, z]
            Gz[:, z] += np.exp(top - CD[:, c])[:, :, None, None] * states[:, c]
        if initial_states is not None:
            Gz[:, z] += np.exp(CDm1[:, z])[:, :, None, None] * initial_states
    Y_off = np.einsum("bclhn,bchpn,bclh->bclhp", Cc, Gz, np.exp(A_cumsum))
    return (Y_diag + Y_off).reshape(b, nc * chunk, H, D)[:, :T]


@pytest.mark.parametrize("T,chunk", [(16, 4), (23, 4), (20, 8), (5, 8)])
def test_matches_pages_chunkwise_algorithm(T, chunk):
    x, B, C, dt, A, h0 = problem(5, T=T, h0=True)
    r = oracle.ssd_complex_fwd(x, B, C, dt, A, initial_states=h0)
    ref = pages_chunkwise(x, B, C, dt, A, chunk, initial_states=h0)
    assert rel(r.y, ref) < 1e-11
    assert rel(r.y.real, ref.real) < 1e-11


def test_propagation_window_matters():
    # the off-by-one the page warns about (CD[z] instead of CD[z-1]) is a
    # different function for time-varying dt, and the oracle is not it
    x, B, C, dt, A, _ = problem(6, T=16)
    r = oracle.ssd_complex_fwd(x, B, C, dt, A)
    assert rel(r.y, pages_chunkwise(x, B, C, dt, A, 4)) < 1e-11
    wrong = pages_chunkwise(x, B, C, dt, A, 4, window_off_by_one=True)
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
