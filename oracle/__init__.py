"""The oracle: a plain, slow, CPU implementation of the Mamba-2 SSD forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``libssd``) and its Python binding never import, link or call it, and
the two share no code: the only module both sides use is the seeded input
generator, which holds none of the method's arithmetic.

Contents
--------
* ``ssd_fwd``            -- the fp64 sequential recurrence (``ssd_ref.c``),
                            Mamba-3-Lite "SSD Reference", section "Math: the
                            recurrence both functions implement", plus dt bias,
                            groups, D skip, SiLU gate, initial/final states and
                            packed sequences.
* ``varlen_chunk_meta``  -- the sequence-aligned chunk table, pure Python ints.
* ``chunk_cumsum``       -- within-chunk cumulative log-decay, SSD Reference
                            section "Chunking and the discretized log-decay".
* ``bmm_chunk``          -- C.B^T per chunk and group, SSD Reference
                            "Algorithm and tensor-shape contract", step 4.
* ``chunk_states``       -- each chunk's end state from a zero start, SSD
                            Reference "Algorithm and tensor-shape contract",
                            step 6 (computed by running the recurrence on the
                            chunk alone).
* ``carry_in_states``    -- the state entering every chunk, SSD Reference
                            "Inter-chunk propagation" (computed as the
                            recurrence's state at the chunk boundary).
* ``state_passing``      -- the chunk-level recurrence applied to given chunk
                            states, SSD Reference "Inter-chunk propagation".
* ``ssd_fwd_stored_states`` -- the chunked forward with its per-chunk states
                            stored in a narrower type (bf16), rounded where they
                            are stored (vLLM PR 27299 "Purpose": the state dtype).
* ``round_to_bf16``      -- round to the nearest bfloat16, ties to even.
* ``ssd_complex_fwd``    -- the fp64 sequential recurrence with a complex
                            per-head A (``ssd_ref_complex.c``), SSD Reference
                            "Math" with "_discretise" exp(softplus(dt) A).
* ``ssd_bwd``            -- the reverse-mode gradient of ``ssd_fwd`` (every input,
                            the initial state included), the adjoint recurrence
                            taken token by token in reverse (``ssd_ref.c``,
                            ``ssd_ref_bwd``); the backward stages of mamba PR 1012
                            "Measurements", SSD Reference section 6 "The autograd
                            backward contract".

* ``gated_rmsnorm_fwd`` / ``gated_rmsnorm_bwd`` -- the gated RMSNorm after the
                            scan (mamba PR 1012's "gated-LayerNorm"; formula:
                            Mamba-2's gated RMSNorm, gate first), numpy fp64.

All floating-point work is fp64.  Every function here is pinned by the
``-m "not gpu"`` tests against closed forms, special cases and brute force.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_ref.c")
_SRC_COMPLEX = os.path.join(_HERE, "ssd_ref_complex.c")
_LIB = os.path.join(_HERE, "libssd_ref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``ssd_ref.c`` and ``ssd_ref_complex.c`` into ``libssd_ref.so``
    with gcc (fp64, OpenMP).

    ``-ffp-contract=off`` keeps every multiply and add separately rounded, as
    written; the portable ``-march=x86-64-v2`` lets the library built here run
    on any x86-64 host it is copied to.
    """
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-march=x86-64-v2", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", "-std=c99", _SRC, _SRC_COMPLEX, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        lib.ssd_ref_fwd.restype = ctypes.c_int
        lib.ssd_ref_fwd.argtypes = [
            ctypes.c_int64, ctypes.c_int, P(ctypes.c_int64),
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int,
        ]
        lib.ssd_ref_bwd.restype = ctypes.c_int
        lib.ssd_ref_bwd.argtypes = [
            ctypes.c_int64, ctypes.c_int, P(ctypes.c_int64),
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int,
        ]
        lib.ssd_ref_num_chunks.restype = ctypes.c_int64
        lib.ssd_ref_num_chunks.argtypes = [ctypes.c_int, P(ctypes.c_int64), ctypes.c_int]
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _packed(a, lead):
    """(b, T, ...) -> (b*T, ...) when the batch axis is present."""
    if a is None:
        return None
    return a.reshape((-1,) + a.shape[lead:])


@dataclass
class FwdResult:
    y: np.ndarray                 # same leading layout as x
    final_states: np.ndarray      # (nseq or b, H, P, N)
    chunk_end_states: np.ndarray | None  # (nchunks, H, P, N) or None


def ssd_fwd(x, B, C, dt, A, dt_bias=None, D=None, z=None, initial_states=None,
            cu_seqlens=None, dt_softplus=True, dt_limit=None, chunk_size=0,
            threads=None, input_dt=False) -> FwdResult:
    """Run the fp64 recurrence.

    Batch mode: x (b, T, H, P), B and C (b, T, G, N), dt (b, T, H), z like x,
    initial_states (b, H, P, N).  Packed mode (``cu_seqlens`` given): the same
    tensors without the batch axis, i.e. x (T, H, P), with sequence i owning
    tokens [cu[i], cu[i+1]); initial_states (nseq, H, P, N).

    ``dt_limit=(lo, hi)`` clamps the step size after softplus.
    ``input_dt=True`` scales the input term by the step size,
    S = exp(delta A) S + delta x (outer) B (the D skip keeps the raw x).  With
    ``chunk_size > 0`` the state after the last token of every sequence-aligned
    chunk is returned as ``chunk_end_states`` (logical chunk order:
    sequence-major, in token order inside a sequence).
    """
    x = _f64(x)
    if cu_seqlens is None:
        b, T = x.shape[0], x.shape[1]
        cu = np.arange(b + 1, dtype=np.int64) * T
        lead = 2
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        lead = 1
    H, P = x.shape[lead], x.shape[lead + 1]
    Bf, Cf = _f64(B), _f64(C)
    G, N = Bf.shape[lead], Bf.shape[lead + 1]
    xs, Bs, Cs = _packed(x, lead), _packed(Bf, lead), _packed(Cf, lead)
    dts = _packed(_f64(dt), lead)
    zs = _packed(_f64(z), lead) if z is not None else None
    ntok = xs.shape[0]
    nseq = len(cu) - 1
    A_ = _f64(np.broadcast_to(np.asarray(A, dtype=np.float64), (H,)))
    bias = _f64(dt_bias)
    D_ = _f64(D)
    h0 = _f64(initial_states)
    y = np.empty((ntok, H, P), dtype=np.float64)
    hfin = np.empty((nseq, H, P, N), dtype=np.float64)
    lib = _load()
    cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    hch = None
    if chunk_size > 0:
        nck = lib.ssd_ref_num_chunks(nseq, cu_p, int(chunk_size))
        hch = np.empty((nck, H, P, N), dtype=np.float64)
    clamp = 0 if dt_limit is None else 1
    lo, hi = (0.0, math.inf) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    rc = lib.ssd_ref_fwd(ntok, nseq, cu_p, H, P, N, G, _ptr(xs), _ptr(Bs), _ptr(Cs),
                         _ptr(dts), _ptr(A_), _ptr(bias), _ptr(D_), _ptr(zs), _ptr(h0),
                         1 if dt_softplus else 0, clamp, lo, hi, 1 if input_dt else 0,
                         int(chunk_size), _ptr(y), _ptr(hfin), _ptr(hch),
                         int(threads or 0))
    if rc != 0:
        raise ValueError(f"ssd_ref_fwd failed with code {rc}")
    return FwdResult(y.reshape(x.shape), hfin, hch)


@dataclass
class BwdResult:
    dx: np.ndarray                # like x
    dB: np.ndarray                # like B (summed over the heads of each group)
    dC: np.ndarray                # like C (summed over the heads of each group)
    ddt: np.ndarray               # like dt: gradient w.r.t. the raw dt
    dA: np.ndarray                # (H,)
    ddt_bias: np.ndarray          # (H,)
    dD: np.ndarray | None         # (H,), None without D
    dz: np.ndarray | None         # like z, None without z
    dinitial_states: np.ndarray   # (nseq or b, H, P, N)


def ssd_bwd(x, B, C, dt, A, dout, dt_bias=None, D=None, z=None, initial_states=None,
            dfinal_states=None, cu_seqlens=None, dt_softplus=True, dt_limit=None,
            threads=None, input_dt=False) -> BwdResult:
    """Gradient of L = sum(dout * y) + sum(dfinal_states * final_states).

    Arguments as ``ssd_fwd``; ``dout`` is shaped like x and ``dfinal_states``
    like the final states (None = zero).  ``ddt`` is the gradient with respect
    to the raw dt (before bias and softplus); where the clamp of ``dt_limit``
    is active it is zero.  A missing initial state is a zero one, and its
    gradient is still returned.
    """
    x = _f64(x)
    if cu_seqlens is None:
        b, T = x.shape[0], x.shape[1]
        cu = np.arange(b + 1, dtype=np.int64) * T
        lead = 2
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        lead = 1
    H, P = x.shape[lead], x.shape[lead + 1]
    Bf, Cf = _f64(B), _f64(C)
    G, N = Bf.shape[lead], Bf.shape[lead + 1]
    xs, Bs, Cs = _packed(x, lead), _packed(Bf, lead), _packed(Cf, lead)
    dts = _packed(_f64(dt), lead)
    zs = _packed(_f64(z), lead) if z is not None else None
    dos = _packed(_f64(dout), lead)
    ntok = xs.shape[0]
    nseq = len(cu) - 1
    A_ = _f64(np.broadcast_to(np.asarray(A, dtype=np.float64), (H,)))
    bias, D_, h0, dfin = _f64(dt_bias), _f64(D), _f64(initial_states), _f64(dfinal_states)
    dx = np.empty((ntok, H, P))
    dB = np.empty((ntok, G, N))
    dC = np.empty((ntok, G, N))
    ddt = np.empty((ntok, H))
    dA = np.empty(H)
    dbias = np.empty(H)
    dD = np.empty(H) if D is not None else None
    dz = np.empty((ntok, H, P)) if z is not None else None
    dh0 = np.empty((nseq, H, P, N))
    clamp = 0 if dt_limit is None else 1
    lo, hi = (0.0, math.inf) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    lib = _load()
    cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = lib.ssd_ref_bwd(ntok, nseq, cu_p, H, P, N, G, _ptr(xs), _ptr(Bs), _ptr(Cs),
                         _ptr(dts), _ptr(A_), _ptr(bias), _ptr(D_), _ptr(zs), _ptr(h0),
                         1 if dt_softplus else 0, clamp, lo, hi, 1 if input_dt else 0,
                         _ptr(dos), _ptr(dfin),
                         _ptr(dx), _ptr(dB), _ptr(dC), _ptr(ddt), _ptr(dA), _ptr(dbias),
                         _ptr(dD), _ptr(dz), _ptr(dh0), int(threads or 0))
    if rc != 0:
        raise ValueError(f"ssd_ref_bwd failed with code {rc}")
    shp = lambda a, like: a.reshape(np.shape(like))
    return BwdResult(shp(dx, x), shp(dB, Bf), shp(dC, Cf), shp(ddt, dt), dA, dbias, dD,
                     None if dz is None else shp(dz, z), dh0)


# --------------------------------------------------------------------------
# Sequence-aligned chunk table (pure Python integers).
# --------------------------------------------------------------------------

@dataclass
class ChunkMeta:
    nchunks: int                 # number of logical chunks K
    seq: list                    # seq[j]   sequence that chunk j belongs to
    start: list                  # start[j] first token of chunk j
    length: list                 # length[j] tokens in chunk j (1..C)
    first_chunk: list            # first_chunk[i] first chunk of sequence i; [nseq] = K


def varlen_chunk_meta(cu_seqlens, chunk_size) -> ChunkMeta:
    """Split every sequence of a packed batch into chunks of ``chunk_size``.

    Sequence i (tokens [cu[i], cu[i+1])) of length L_i is cut at multiples of
    the chunk size counted from its own first token, giving ceil(L_i / C)
    chunks; an empty sequence gets none.  Chunks are numbered sequence by
    sequence.  This is the chunk grid of the SSD Reference ("Padding rule",
    "Chunking") applied to each sequence separately, so that no chunk straddles
    a sequence boundary and the state can restart there (vLLM PR 27299,
    continuous batching).
    """
    cu = [int(v) for v in cu_seqlens]
    C = int(chunk_size)
    seq, start, length, first = [], [], [], []
    for i in range(len(cu) - 1):
        first.append(len(seq))
        L = cu[i + 1] - cu[i]
        k = 0
        while k * C < L:
            seq.append(i)
            start.append(cu[i] + k * C)
            length.append(min(C, L - k * C))
            k += 1
    first.append(len(seq))
    return ChunkMeta(len(seq), seq, start, length, first)


def batch_chunk_meta(batch, seqlen, chunk_size) -> ChunkMeta:
    """The chunk table of ``batch`` equal sequences of ``seqlen`` tokens."""
    return varlen_chunk_meta([i * seqlen for i in range(batch + 1)], chunk_size)


# --------------------------------------------------------------------------
# Stage intermediates.  Tokens are addressed on the packed axis (b*T for
# batch mode), and chunks by their logical id j from the chunk table.
# --------------------------------------------------------------------------

def softplus(u):
    """log(1 + e^u) in the overflow-free form max(u,0) + log1p(exp(-|u|))."""
    u = np.asarray(u, dtype=np.float64)
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def step_size(dt, dt_bias=None, dt_softplus=True, dt_limit=None):
    """delta = softplus(dt + dt_bias), optionally clamped (per token, per head)."""
    u = np.asarray(dt, dtype=np.float64)
    if dt_bias is not None:
        u = u + np.asarray(dt_bias, dtype=np.float64)
    d = softplus(u) if dt_softplus else u
    if dt_limit is not None:
        d = np.minimum(np.maximum(d, dt_limit[0]), dt_limit[1])
    return d


def chunk_cumsum(dt, A, meta: ChunkMeta, chunk_size, dt_bias=None, dt_softplus=True,
                 dt_limit=None):
    """Within-chunk inclusive cumulative sum of the log-decay a = delta * A.

    dt is (ntok, H) on the packed token axis.  Returns (K, H, C) fp64.  A chunk
    shorter than C is treated as if the missing positions had a = 0, so those
    positions repeat the value at the chunk's last token.
    """
    dt = np.asarray(dt, dtype=np.float64)
    H = dt.shape[1]
    C = int(chunk_size)
    a = step_size(dt, dt_bias, dt_softplus, dt_limit) * np.asarray(A, dtype=np.float64)[None, :]
    out = np.zeros((meta.nchunks, H, C), dtype=np.float64)
    for j in range(meta.nchunks):
        s, L = meta.start[j], meta.length[j]
        seg = np.zeros((C, H), dtype=np.float64)
        seg[:L] = a[s:s + L]
        out[j] = np.cumsum(seg, axis=0).T
    return out


def bmm_chunk(Cm, Bm, meta: ChunkMeta, chunk_size):
    """CB[j, g, l, s] = sum_n C[start_j + l, g, n] * B[start_j + s, g, n].

    Cm, Bm are (ntok, G, N).  Returns (K, G, C, C) fp64; rows or columns past a
    short chunk's end are zero.
    """
    Cm = np.asarray(Cm, dtype=np.float64)
    Bm = np.asarray(Bm, dtype=np.float64)
    G = Cm.shape[1]
    Cs = int(chunk_size)
    out = np.zeros((meta.nchunks, G, Cs, Cs), dtype=np.float64)
    for j in range(meta.nchunks):
        s, L = meta.start[j], meta.length[j]
        for g in range(G):
            out[j, g, :L, :L] = np.matmul(Cm[s:s + L, g, :], Bm[s:s + L, g, :].T)
    return out


def _chunk_cut(meta: ChunkMeta):
    """cu_seqlens whose sequences are exactly the chunks of ``meta``."""
    cuts = [meta.start[j] for j in range(meta.nchunks)]
    if meta.nchunks:
        cuts.append(meta.start[-1] + meta.length[-1])
    else:
        cuts.append(0)
    return np.asarray(cuts, dtype=np.int64)


def chunk_states(x, Bm, dt, A, meta: ChunkMeta, dt_bias=None, dt_softplus=True,
                 dt_limit=None, threads=None, input_dt=False):
    """Each chunk's end state with a zero state entering the chunk: (K, H, P, N).

    Computed by running the recurrence on every chunk as its own sequence; x is
    (ntok, H, P), Bm (ntok, G, N), dt (ntok, H), all on the packed token axis.
    Tokens that belong to no chunk (between packed sequences there are none)
    are never read.
    """
    x = np.asarray(x, dtype=np.float64)
    H, P = x.shape[1], x.shape[2]
    N = np.asarray(Bm).shape[2]
    if meta.nchunks == 0:
        return np.zeros((0, H, P, N))
    cu = _chunk_cut(meta)
    lo, hi = int(cu[0]), int(cu[-1])
    Cz = np.zeros_like(np.asarray(Bm, dtype=np.float64)[lo:hi])
    r = ssd_fwd(x[lo:hi], np.asarray(Bm)[lo:hi], Cz, np.asarray(dt)[lo:hi], A,
                dt_bias=dt_bias, cu_seqlens=cu - lo, dt_softplus=dt_softplus,
                dt_limit=dt_limit, threads=threads, input_dt=input_dt)
    return r.final_states


def carry_in_states(chunk_end_states, meta: ChunkMeta, initial_states=None):
    """State entering every chunk: (K, H, P, N).

    The first chunk of sequence i starts from initial_states[i] (or zero); every
    other chunk starts from the state after the last token of the chunk before
    it, i.e. ``chunk_end_states[j - 1]`` from a full recurrence run.
    """
    K = meta.nchunks
    shp = chunk_end_states.shape[1:]
    out = np.zeros((K,) + shp, dtype=np.float64)
    for j in range(K):
        i = meta.seq[j]
        if j == meta.first_chunk[i]:
            if initial_states is not None:
                out[j] = np.asarray(initial_states, dtype=np.float64)[i]
        else:
            out[j] = chunk_end_states[j - 1]
    return out


def state_passing(S, cs, meta: ChunkMeta, initial_states=None):
    """The inter-chunk recurrence on given chunk states (fp64).

    SSD Reference, "Inter-chunk propagation": the state entering chunk z is the
    sum over earlier chunks c of exp(CD[z-1] - CD[c]) S_c plus exp(CD[z-1])
    times the initial state, which is the recurrence
        Hin[first] = h_init (or 0),  Hin[j + 1] = exp(Lambda_j) Hin[j] + S_j
    with Lambda_j = cs[j, :, len_j - 1], restarted at every sequence's first
    chunk.  S is (K, H, P, N), cs (K, H, C).  Returns (Hin (K, H, P, N),
    final (nseq, H, P, N)); an empty sequence's final state is its initial state.
    """
    S = np.asarray(S, dtype=np.float64)
    cs = np.asarray(cs, dtype=np.float64)
    K = meta.nchunks
    nseq = len(meta.first_chunk) - 1
    shp = S.shape[1:]
    Hin = np.zeros((K,) + shp)
    final = np.zeros((nseq,) + shp)
    for i in range(nseq):
        cur = (np.zeros(shp) if initial_states is None
               else np.asarray(initial_states, dtype=np.float64)[i].copy())
        for j in range(meta.first_chunk[i], meta.first_chunk[i + 1]):
            Hin[j] = cur
            lam = cs[j, :, meta.length[j] - 1]
            cur = np.exp(lam)[:, None, None] * cur + S[j]
        final[i] = cur
    return Hin, final


def round_to_bf16(a):
    """Round to the nearest bfloat16 value, ties to even, returned as fp64.

    The value is first rounded to the nearest float32 (numpy's conversion), then
    its 16 low bits are rounded off: add 0x7FFF plus the lowest kept bit, clear
    the low half.  Infinities and NaN are passed through unchanged.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    keep = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    special = ~np.isfinite(f)
    out[special] = f[special]
    return out


def ssd_fwd_stored_states(x, B, C, dt, A, dt_bias=None, D=None, z=None,
                          initial_states=None, cu_seqlens=None, chunk_size=128,
                          dt_softplus=True, dt_limit=None, input_dt=False,
                          state_dtype="bf16", threads=None) -> FwdResult:
    """The chunked forward with its per-chunk states stored in ``state_dtype``.

    vLLM PR 27299 ("Purpose") names the state dtype as an axis of the SSD
    stages: the states the chunk-state stage writes and the state-passing
    stage reads and writes are held in that type.  With a narrow type the
    result is no longer the plain recurrence's, so this follows the chunked
    algorithm's steps (SSD Reference, "Intra-chunk outputs and per-chunk
    states", "Inter-chunk propagation", "Readout") and rounds exactly where a
    value is stored:
      1. every chunk's end state from a zero start, S_j (fp64), stored rounded;
      2. the inter-chunk recurrence Hin[j+1] = exp(Lambda_j) Hin[j] + S_j over
         the stored S_j, carried in full precision (a register value); each
         carry-in Hin[j] is stored rounded; the final state is the carried
         value, not rounded (final states are float32 outputs);
      3. every chunk's outputs from its stored carry-in: the recurrence run on
         the chunk alone from that state (= the intra-chunk part plus the
         readout of the carried state, by linearity).
    ``state_dtype`` is "bf16" (round to nearest even) or "f32" (round to the
    nearest float32).  Arguments and layouts as ``ssd_fwd``.
    """
    if state_dtype == "bf16":
        rnd = round_to_bf16
    elif state_dtype == "f32":
        rnd = lambda a: np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    else:
        raise ValueError(f"state_dtype {state_dtype!r}")
    x = _f64(x)
    if cu_seqlens is None:
        b, T = x.shape[0], x.shape[1]
        cu = np.arange(b + 1, dtype=np.int64) * T
        lead = 2
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        lead = 1
    xs, Bs, Cs = _packed(x, lead), _packed(_f64(B), lead), _packed(_f64(C), lead)
    dts = _packed(_f64(dt), lead)
    zs = _packed(_f64(z), lead) if z is not None else None
    meta = varlen_chunk_meta(cu, chunk_size)
    S = chunk_states(xs, Bs, dts, A, meta, dt_bias=dt_bias, dt_softplus=dt_softplus,
                     dt_limit=dt_limit, threads=threads, input_dt=input_dt)
    cs = chunk_cumsum(dts, A, meta, chunk_size, dt_bias=dt_bias, dt_softplus=dt_softplus,
                      dt_limit=dt_limit)
    Hin, final = state_passing(rnd(S), cs, meta, initial_states)
    H, P = xs.shape[1], xs.shape[2]
    y = np.zeros((xs.shape[0], H, P))
    if meta.nchunks:
        cut = _chunk_cut(meta)
        lo, hi = int(cut[0]), int(cut[-1])
        r = ssd_fwd(xs[lo:hi], Bs[lo:hi], Cs[lo:hi], dts[lo:hi], A, dt_bias=dt_bias, D=D,
                    z=None if zs is None else zs[lo:hi], initial_states=rnd(Hin),
                    cu_seqlens=cut - lo, dt_softplus=dt_softplus, dt_limit=dt_limit,
                    threads=threads, input_dt=input_dt)
        y[lo:hi] = r.y
    return FwdResult(y.reshape(x.shape), final, None)


# --------------------------------------------------------------------------
# The complex-A scan (ssd_ref_complex.c).
# --------------------------------------------------------------------------

@dataclass
class ComplexResult:
    y: np.ndarray                 # complex128, like x
    final_states: np.ndarray      # complex128, (nseq or b, H, D, N)


def ssd_complex_fwd(x, B, C, dt, A, initial_states=None, cu_seqlens=None,
                    threads=None) -> ComplexResult:
    """Run the fp64 complex recurrence (SSD Reference, "Math" with complex A).

    Batch mode: x (b, T, H, D), B and C (b, T, H, N) complex, dt (b, T, H) real,
    A (H,) complex, initial_states (b, H, D, N) complex.  Packed mode: the same
    without the batch axis plus ``cu_seqlens``.  Returns the full complex
    output and the final states in the (D, N) layout.
    """
    x = np.asarray(x)
    if cu_seqlens is None:
        b, T = x.shape[0], x.shape[1]
        cu = np.arange(b + 1, dtype=np.int64) * T
        lead = 2
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        lead = 1
    H, D = x.shape[lead], x.shape[lead + 1]
    N = np.shape(B)[lead + 1]

    def cplx(a):
        return None if a is None else np.ascontiguousarray(
            np.asarray(a, dtype=np.complex128)).view(np.float64)

    xs = cplx(np.reshape(x, (-1, H, D)))
    Bs = cplx(np.reshape(B, (-1, H, N)))
    Cs = cplx(np.reshape(C, (-1, H, N)))
    dts = np.ascontiguousarray(np.reshape(np.asarray(dt, dtype=np.float64), (-1, H)))
    A_ = cplx(np.broadcast_to(np.asarray(A, dtype=np.complex128), (H,)))
    h0 = cplx(initial_states)
    ntok = xs.shape[0]
    nseq = len(cu) - 1
    y = np.empty((ntok, H, D), dtype=np.complex128)
    hfin = np.empty((nseq, H, D, N), dtype=np.complex128)
    lib = _load()
    f = lib.ssd_ref_complex_fwd
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int,
                  ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 8 + [ctypes.c_int]
    rc = f(ntok, nseq, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, D, N, _ptr(xs),
           _ptr(Bs), _ptr(Cs), _ptr(dts), _ptr(A_), _ptr(h0), _ptr(y.view(np.float64)),
           _ptr(hfin.view(np.float64)), int(threads or 0))
    if rc != 0:
        raise ValueError(f"ssd_ref_complex_fwd failed with code {rc}")
    return ComplexResult(y.reshape(x.shape), hfin)


# ------------------------------------------------------------------ gated RMSNorm
#
# The step after the scan in the Mamba-2 mixer: the "gated-LayerNorm" whose
# backward mamba PR 1012 times ("Summary", "Measurements": layer_norm_bwd).  The
# pages do not write its formula; the reading taken is Mamba-2's gated RMSNorm
# with the gate applied before the norm, over contiguous channel groups of the
# flattened (H, P) axis:
#     g   = y * silu(z)                 (z absent: g = y)
#     r   = 1 / sqrt(mean_group(g^2) + eps)
#     out = g * r * weight

@dataclass
class NormResult:
    out: np.ndarray      # float64, shaped like y
    rstd: np.ndarray     # float64, (..., H * P // group_size)


def _norm_groups(a, group_size):
    lead = a.shape[:-2]
    width = a.shape[-2] * a.shape[-1]
    if width % group_size != 0:
        raise ValueError("group_size must divide H * P")
    return a.reshape(lead + (width // group_size, group_size))


def gated_rmsnorm_fwd(y, z, weight, group_size, eps=1e-5) -> NormResult:
    """fp64 forward of the gated RMSNorm.  y, z (..., H, P); weight (H * P,)."""
    y = np.asarray(y, dtype=np.float64)
    g = y if z is None else y * (np.asarray(z, dtype=np.float64) /
                                 (1.0 + np.exp(-np.asarray(z, dtype=np.float64))))
    gg = _norm_groups(g, group_size)
    ms = np.mean(gg * gg, axis=-1)
    r = 1.0 / np.sqrt(ms + eps)
    xhat = gg * r[..., None]
    w = _norm_groups(np.asarray(weight, dtype=np.float64).reshape(y.shape[-2:]), group_size)
    out = (xhat * w).reshape(y.shape)
    return NormResult(out, r)


@dataclass
class NormGrads:
    dy: np.ndarray
    dz: np.ndarray | None
    dweight: np.ndarray   # (H * P,)


def gated_rmsnorm_bwd(y, z, weight, dout, group_size, eps=1e-5) -> NormGrads:
    """fp64 gradient of sum(dout * out) with respect to y, z and weight.

    With xhat = g r:  dxhat = dout w;  dg = r (dxhat - xhat mean_group(dxhat xhat));
    dy = dg silu(z);  dz = dg y sigma(z) (1 + z (1 - sigma(z)));  dweight = sum over
    tokens of dout xhat.
    """
    y = np.asarray(y, dtype=np.float64)
    shape = y.shape
    if z is not None:
        z = np.asarray(z, dtype=np.float64)
        sig = 1.0 / (1.0 + np.exp(-z))
        g = y * z * sig
    else:
        g = y
    gg = _norm_groups(g, group_size)
    r = 1.0 / np.sqrt(np.mean(gg * gg, axis=-1) + eps)
    xhat = gg * r[..., None]
    w = _norm_groups(np.asarray(weight, dtype=np.float64).reshape(shape[-2:]), group_size)
    do = _norm_groups(np.asarray(dout, dtype=np.float64), group_size)
    dxhat = do * w
    dg = r[..., None] * (dxhat - xhat * np.mean(dxhat * xhat, axis=-1, keepdims=True))
    dg = dg.reshape(shape)
    dweight = np.sum((do * xhat).reshape((-1,) + shape[-2:]), axis=0).reshape(-1)
    if z is None:
        return NormGrads(dg, None, dweight)
    dy = dg * z * sig
    dz = dg * y * sig * (1.0 + z * (1.0 - sig))
    return NormGrads(dy, dz, dweight)
