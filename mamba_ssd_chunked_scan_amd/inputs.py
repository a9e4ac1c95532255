"""Seeded synthetic inputs for the SSD forward pass.

This module is the only code that both the oracle side (tests, the CPU
baseline) and the HIP side (tests, the benchmark) use.  It draws random
tensors and rounds them to the storage precision; it contains none of the
scan's arithmetic.

Workload shapes follow the pages' benchmark dimensions (Nemotron-Nano: 64
heads x 64, d_state 128, 8 groups, chunk 128, seq 8192, mamba PR 1012
"Measurements"; granite-4.0-h-small: 128 heads x 64, 1 group, d_state 128,
vLLM PR 27299 microbenchmark table).  No dataset is involved anywhere: every
page's SSD measurement is a synthetic-tensor kernel benchmark.

Recipe (one ``numpy.random.Generator(PCG64(seed))``, drawn in this order):
  1. x      ~ N(0, 1)                       (b, T, H, P)
  2. B      ~ N(0, 1)                       (b, T, G, N)
  3. C      ~ N(0, 1)                       (b, T, G, N)
  4. dt     ~ N(0, 1)                       (b, T, H)     raw, before bias
  5. u_h    = exp(U(ln 1e-3, ln 1e-1)),  dt_bias_h = log(expm1(u_h))
     so that softplus(dt_bias_h) = u_h lies in [1e-3, 0.1]
  6. A_h    = -exp(U(ln 1, ln 16))          (H)
  7. D_h    ~ N(0, 1)                       (H)
  8. z      ~ N(0, 1)                       (b, T, H, P)   if gated
For bf16 workloads x, B, C, dt and z are rounded to bf16 (round to nearest
even) and kept as float32 arrays holding exactly the bf16 values; A, dt_bias
and D stay float32.  The initial state is zero unless a test asks otherwise.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def round_bf16(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


@dataclass
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    chunk_size: int
    dtype: str = "bf16"          # storage dtype of x, B, C, dt, z: "bf16" or "f32"
    has_D: bool = True
    has_z: bool = True
    seed: int = 0
    nseq: int = 0                # > 0: packed varlen batch of nseq sequences (batch must be 1)
    seqlens: tuple | None = None  # explicit lengths for the packed batch
    state_dtype: str | None = None  # storage dtype of inter-chunk states (None = dtype)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The five configurations of the workload table.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 4, 16, 1, 16, 64, dtype="f32", has_D=True,
                     has_z=False, seed=1000),
    "granite": Workload("granite", 1, 4096, 128, 64, 1, 128, 128, seed=1001),
    "nemotron": Workload("nemotron", 1, 8192, 64, 64, 8, 128, 128, seed=1002),
    "nemotron_varlen": Workload("nemotron_varlen", 1, 8192, 64, 64, 8, 128, 128,
                                seed=1002, nseq=8),
    "longctx": Workload("longctx", 1, 65536, 80, 64, 1, 128, 256, has_z=False,
                        seed=1003),
    # the forward + backward shape of cudnn-frontend PR 1133 (batch 2, seq 2048,
    # 64 heads, head and state dim 64, one group), gated and ungated; timed with
    # 128-token chunks (the result does not depend on the chunk length)
    "cudnn_gated": Workload("cudnn_gated", 2, 2048, 64, 64, 1, 64, 128, seed=1004),
    "cudnn_ungated": Workload("cudnn_ungated", 2, 2048, 64, 64, 1, 64, 128, has_z=False,
                              seed=1005),
}


@dataclass
class Inputs:
    x: np.ndarray
    B: np.ndarray
    C: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    dt_bias: np.ndarray
    D: np.ndarray | None
    z: np.ndarray | None
    cu_seqlens: np.ndarray | None = None
    initial_states: np.ndarray | None = None
    extra: dict = field(default_factory=dict)


def random_cu_seqlens(rng, total, nseq):
    """nseq - 1 distinct cut points drawn uniformly from 1..total-1, sorted."""
    cuts = np.sort(rng.choice(np.arange(1, total), size=nseq - 1, replace=False))
    return np.concatenate([[0], cuts, [total]]).astype(np.int32)


def make_inputs(w: Workload, seed: int | None = None) -> Inputs:
    """Draw the inputs of workload ``w`` (see the module docstring for the recipe).

    For a packed batch (``w.nseq > 0``) the arrays have no batch axis: x is
    (T, H, P), and ``cu_seqlens`` holds nseq + 1 int32 offsets.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    b, T, H, P, G, N = w.batch, w.seqlen, w.nheads, w.headdim, w.ngroups, w.dstate
    x = rng.standard_normal((b, T, H, P), dtype=np.float32)
    B = rng.standard_normal((b, T, G, N), dtype=np.float32)
    C = rng.standard_normal((b, T, G, N), dtype=np.float32)
    dt = rng.standard_normal((b, T, H), dtype=np.float32)
    u = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=H))
    dt_bias = (u + np.log(-np.expm1(-u))).astype(np.float32)
    A = (-np.exp(rng.uniform(np.log(1.0), np.log(16.0), size=H))).astype(np.float32)
    D = rng.standard_normal(H, dtype=np.float32) if w.has_D else None
    z = rng.standard_normal((b, T, H, P), dtype=np.float32) if w.has_z else None
    if w.dtype == "bf16":
        x, B, C, dt = round_bf16(x), round_bf16(B), round_bf16(C), round_bf16(dt)
        if z is not None:
            z = round_bf16(z)
    cu = None
    if w.nseq > 0 or w.seqlens is not None:
        if b != 1:
            raise ValueError("a packed batch has batch == 1")
        if w.seqlens is not None:
            lens = np.asarray(w.seqlens, dtype=np.int64)
            if int(lens.sum()) != T:
                raise ValueError("seqlens must sum to seqlen")
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        else:
            cu = random_cu_seqlens(rng, T, w.nseq)
        x, B, C, dt = x[0], B[0], C[0], dt[0]
        if z is not None:
            z = z[0]
    return Inputs(x, B, C, dt, A, dt_bias, D, z, cu)


def edge_seqlens(chunk_size: int, total: int) -> tuple:
    """Sequence lengths around chunk edges (1, C-1, C, C+1, 2C+3, ...), padded to total."""
    C = chunk_size
    lens = [1, C - 1, C, C + 1, 2 * C + 3, 3, 2 * C, 5 * C - 1]
    s = sum(lens)
    if s > total:
        raise ValueError("total too small for the edge-length pattern")
    lens.append(total - s)
    return tuple(lens)


# ------------------------------------------------------------------ complex A
#
# The complex-A scan of the Mamba-3-Lite SSD Reference page.  Its production
# shape is the page's 434M configuration (batch 8, seq 2048, chunk 64, 16 heads,
# head dim 64, state dim 64; complex64 throughout, dt float32).  The page's own
# tests draw random complex A, B, C, x and dt; the recipe below keeps the real
# workloads' step-size and decay-rate ranges (the complex call has no dt bias,
# so the per-head offset is folded into dt).  One Generator(PCG64(seed)), in
# this order:
#   1. x  = N(0,1) + i N(0,1)                       (b, T, H, P)  (real part, then imaginary)
#   2. B  = N(0,1) + i N(0,1)                       (b, T, H, N)
#   3. C  = N(0,1) + i N(0,1)                       (b, T, H, N)
#   4. dt = N(0,1) + log(expm1(u_h)),  u_h = exp(U(ln 1e-3, ln 0.1))   (b, T, H)
#      so softplus of the per-head offset is u_h
#   5. A_h = -exp(U(ln 1, ln 16)) + i U(-pi, pi)    (H)
#   6. initial state N(0,1) + i N(0,1)              (b, H, P, N)  if asked
# Values are rounded to complex64 / float32; the oracle consumes those values.

@dataclass
class ComplexWorkload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    chunk_size: int
    seed: int = 0
    initial_states: bool = False

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


@dataclass
class ComplexInputs:
    x: np.ndarray        # complex64 (b, T, H, P)
    B: np.ndarray        # complex64 (b, T, H, N)
    C: np.ndarray        # complex64 (b, T, H, N)
    dt: np.ndarray       # float32 (b, T, H)
    A: np.ndarray        # complex64 (H,)
    h0: np.ndarray | None  # complex64 (b, H, P, N)


def _cnormal(rng, shape):
    re = rng.standard_normal(shape, dtype=np.float32)
    im = rng.standard_normal(shape, dtype=np.float32)
    out = np.empty(shape, dtype=np.complex64)
    out.real = re
    out.imag = im
    return out


def make_complex_inputs(w: ComplexWorkload, seed: int | None = None) -> ComplexInputs:
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    b, T, H, P, N = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate
    x = _cnormal(rng, (b, T, H, P))
    B = _cnormal(rng, (b, T, H, N))
    C = _cnormal(rng, (b, T, H, N))
    dt = rng.standard_normal((b, T, H), dtype=np.float32)
    u = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), H))
    dt = (dt + np.log(np.expm1(u)).astype(np.float32)).astype(np.float32)
    A = (-np.exp(rng.uniform(np.log(1.0), np.log(16.0), H))
         + 1j * rng.uniform(-np.pi, np.pi, H)).astype(np.complex64)
    h0 = _cnormal(rng, (b, H, P, N)) if w.initial_states else None
    return ComplexInputs(x, B, C, dt, A, h0)


COMPLEX_WORKLOADS = {
    "complex_tiny": ComplexWorkload("complex_tiny", 2, 300, 3, 32, 32, 64, seed=2000,
                                    initial_states=True),
    # SSD Reference (Mamba-3-Lite) 434M configuration: B=8, T=2048, C=64, H=16, D=64, N=64
    "complex_434m": ComplexWorkload("complex_434m", 8, 2048, 16, 64, 64, 64, seed=2001),
}
