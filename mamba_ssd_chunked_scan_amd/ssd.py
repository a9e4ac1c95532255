"""Thin Python binding of libssd (ctypes).

Argument marshalling only: torch supplies device memory (``data_ptr()``),
strides and the current stream; every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/ssd.h``.  There is no fallback:
if ``libssd.so`` has not been built, or a call fails, an exception is raised.

Function names follow the C calls: ``ssd_chunk_cumsum``, ``ssd_bmm_chunk``,
``ssd_chunk_state``, ``ssd_state_passing``, ``ssd_chunk_scan``,
``ssd_varlen_chunk_meta``, ``ssd_forward``, ``ssd_backward``.  Each takes torch
tensors and returns the tensors it wrote.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")

SSD_OK = 0
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE",
          4: "SSD_ERR_STRIDE", 5: "SSD_ERR_UNSUPPORTED", 6: "SSD_ERR_WORKSPACE", 7: "SSD_ERR_HIP"}
F32, BF16 = 0, 1
ALGO = {"staged": 0, "fused": 1, "auto": 2}


class SSDError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class SsdTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int),
                ("stride", ctypes.c_int64 * 3)]


class SsdProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("nseq", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("chunk_meta", ctypes.c_void_p),
                ("dt_softplus", ctypes.c_int32), ("dt_clamp", ctypes.c_int32),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float),
                ("state_dtype", ctypes.c_int), ("input_dt", ctypes.c_int32)]


class SsdFwdArgs(ctypes.Structure):
    _fields_ = [("x", SsdTensor), ("B", SsdTensor), ("C", SsdTensor), ("dt", SsdTensor),
                ("A", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("D", ctypes.c_void_p),
                ("z", SsdTensor), ("initial_states", ctypes.c_void_p), ("out", SsdTensor),
                ("final_states", ctypes.c_void_p)]


class SsdBwdArgs(ctypes.Structure):
    _fields_ = [("x", SsdTensor), ("B", SsdTensor), ("C", SsdTensor), ("dt", SsdTensor),
                ("A", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("D", ctypes.c_void_p),
                ("z", SsdTensor), ("initial_states", ctypes.c_void_p),
                ("dout", SsdTensor), ("dfinal_states", ctypes.c_void_p),
                ("dx", SsdTensor), ("dB", SsdTensor), ("dC", SsdTensor), ("ddt", SsdTensor),
                ("dz", SsdTensor), ("dA", ctypes.c_void_p), ("ddt_bias", ctypes.c_void_p),
                ("dD", ctypes.c_void_p), ("dinitial_states", ctypes.c_void_p)]


class SsdComplexProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("nseq", ctypes.c_int32), ("cu_seqlens", ctypes.c_void_p)]


class SsdComplexFwdArgs(ctypes.Structure):
    _fields_ = [("x", SsdTensor), ("B", SsdTensor), ("C", SsdTensor), ("dt", SsdTensor),
                ("A", ctypes.c_void_p), ("initial_states", ctypes.c_void_p),
                ("out", SsdTensor), ("out_complex", ctypes.c_int32),
                ("final_states", ctypes.c_void_p)]


class SsdNormArgs(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("group_size", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rstd", ctypes.c_void_p)]


class SsdNormProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("eps", ctypes.c_float)]


_lib = None
EXPORTS = ("ssd_problem_check", "ssd_num_chunks", "ssd_varlen_meta_len", "ssd_workspace_size",
           "ssd_varlen_chunk_meta", "ssd_varlen_chunk_meta_host", "ssd_chunk_cumsum",
           "ssd_bmm_chunk", "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan",
           "ssd_forward", "ssd_forward_fused_static", "ssd_forward_gated_norm",
           "ssd_forward_gated_norm_workspace_size",
           "ssd_backward_workspace_size", "ssd_backward",
           "ssd_backward_ex_workspace_size", "ssd_backward_ex",
           "ssd_complex_problem_check", "ssd_complex_workspace_size", "ssd_complex_forward",
           "ssd_complex_chunk_state", "ssd_complex_state_passing", "ssd_complex_chunk_scan",
           "ssd_gated_rmsnorm_fwd", "ssd_gated_rmsnorm_bwd_workspace_size",
           "ssd_gated_rmsnorm_bwd",
           "ssd_status_string", "ssd_last_error_message", "ssd_version")


def lib():
    """The loaded libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m mamba_ssd_chunked_scan_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, st = ctypes.c_void_p, ctypes.c_int
        L.ssd_problem_check.argtypes = [P(SsdProblem)]
        L.ssd_num_chunks.argtypes = [P(SsdProblem)]
        L.ssd_num_chunks.restype = ctypes.c_int64
        L.ssd_varlen_meta_len.argtypes = [P(SsdProblem)]
        L.ssd_varlen_meta_len.restype = ctypes.c_size_t
        L.ssd_workspace_size.argtypes = [P(SsdProblem), ctypes.c_int, P(ctypes.c_size_t)]
        L.ssd_varlen_chunk_meta.argtypes = [P(SsdProblem), vp, vp]
        L.ssd_varlen_chunk_meta_host.argtypes = [P(SsdProblem), P(ctypes.c_int32),
                                                 P(ctypes.c_int32), ctypes.c_size_t]
        L.ssd_chunk_cumsum.argtypes = [P(SsdProblem), SsdTensor, vp, vp, vp, vp, vp]
        L.ssd_bmm_chunk.argtypes = [P(SsdProblem), SsdTensor, SsdTensor, vp, vp]
        L.ssd_chunk_state.argtypes = [P(SsdProblem), SsdTensor, SsdTensor, vp, vp, vp, vp]
        L.ssd_state_passing.argtypes = [P(SsdProblem), vp, vp, vp, vp, vp, vp]
        L.ssd_chunk_scan.argtypes = [P(SsdProblem), vp, SsdTensor, SsdTensor, vp, vp, vp, vp,
                                     SsdTensor, SsdTensor, vp]
        L.ssd_forward.argtypes = [P(SsdProblem), ctypes.c_int, P(SsdFwdArgs), vp,
                                  ctypes.c_size_t, vp]
        L.ssd_forward_fused_static.argtypes = [P(SsdProblem), P(SsdFwdArgs), vp]
        L.ssd_forward_gated_norm_workspace_size.argtypes = [P(SsdProblem), P(SsdNormArgs),
                                                            P(ctypes.c_size_t)]
        L.ssd_forward_gated_norm.argtypes = [P(SsdProblem), P(SsdFwdArgs), P(SsdNormArgs), vp,
                                             ctypes.c_size_t, vp]
        L.ssd_backward_workspace_size.argtypes = [P(SsdProblem), P(ctypes.c_size_t)]
        L.ssd_backward.argtypes = [P(SsdProblem), P(SsdBwdArgs), vp, ctypes.c_size_t, vp]
        L.ssd_backward_ex_workspace_size.argtypes = [P(SsdProblem), ctypes.c_int, ctypes.c_int,
                                                     P(ctypes.c_size_t)]
        L.ssd_backward_ex.argtypes = [P(SsdProblem), P(SsdBwdArgs), ctypes.c_int, vp,
                                      ctypes.c_size_t, vp]
        L.ssd_complex_problem_check.argtypes = [P(SsdComplexProblem)]
        L.ssd_complex_workspace_size.argtypes = [P(SsdComplexProblem), P(ctypes.c_size_t)]
        L.ssd_complex_forward.argtypes = [P(SsdComplexProblem), P(SsdComplexFwdArgs), vp,
                                          ctypes.c_size_t, vp]
        L.ssd_complex_chunk_state.argtypes = [P(SsdComplexProblem), SsdTensor, SsdTensor,
                                              SsdTensor, vp, vp, vp, vp]
        L.ssd_gated_rmsnorm_fwd.argtypes = [P(SsdNormProblem), SsdTensor, SsdTensor, vp,
                                            SsdTensor, vp, vp]
        L.ssd_gated_rmsnorm_bwd_workspace_size.argtypes = [P(SsdNormProblem), P(ctypes.c_size_t)]
        L.ssd_gated_rmsnorm_bwd.argtypes = [P(SsdNormProblem), SsdTensor, SsdTensor, vp,
                                            SsdTensor, SsdTensor, SsdTensor, vp, vp,
                                            ctypes.c_size_t, vp]
        L.ssd_complex_state_passing.argtypes = [P(SsdComplexProblem), vp, vp, vp, vp, vp, vp]
        L.ssd_complex_chunk_scan.argtypes = [P(SsdComplexProblem), SsdTensor, SsdTensor,
                                             SsdTensor, SsdTensor, vp, vp, SsdTensor,
                                             ctypes.c_int32, vp]
        for name in ("ssd_problem_check", "ssd_workspace_size", "ssd_varlen_chunk_meta",
                     "ssd_varlen_chunk_meta_host", "ssd_chunk_cumsum", "ssd_bmm_chunk",
                     "ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan", "ssd_forward",
                     "ssd_forward_fused_static", "ssd_forward_gated_norm",
                     "ssd_forward_gated_norm_workspace_size",
                     "ssd_backward_workspace_size", "ssd_backward",
                     "ssd_backward_ex_workspace_size", "ssd_backward_ex",
                     "ssd_complex_problem_check", "ssd_complex_workspace_size",
                     "ssd_complex_forward", "ssd_complex_chunk_state",
                     "ssd_complex_state_passing", "ssd_complex_chunk_scan",
                     "ssd_gated_rmsnorm_fwd", "ssd_gated_rmsnorm_bwd_workspace_size",
                     "ssd_gated_rmsnorm_bwd"):
            getattr(L, name).restype = st
        L.ssd_status_string.argtypes = [ctypes.c_int]
        L.ssd_status_string.restype = ctypes.c_char_p
        L.ssd_last_error_message.restype = ctypes.c_char_p
        L.ssd_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc):
    if rc != SSD_OK:
        raise SSDError(rc, lib().ssd_last_error_message().decode())


# ------------------------------------------------------------------ marshalling

def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise SSDError(3, f"unsupported dtype {t}")


def tensor_arg(t: torch.Tensor | None, packed: bool = False) -> SsdTensor:
    """ssd_tensor of a (b, T, X, Y) / (b, T, X) tensor, or (T, ...) when packed.

    The innermost dimension must be contiguous for the 4-D roles; for the 3-D dt
    role all three strides are passed.
    """
    s = SsdTensor()
    if t is None or t.numel() == 0:
        # absent, or empty (no tokens): no memory to point at
        s.data = None
        s.dtype = F32 if t is None else _dtype_code(t.dtype)
        return s
    s.data = t.data_ptr()
    s.dtype = _dtype_code(t.dtype)
    st = list(t.stride())
    if packed:
        st = [0] + st
    if len(st) == 4:
        if st[3] != 1 and t.shape[-1 - 0] > 1:
            raise SSDError(4, "innermost dimension must be contiguous")
        outer = st[:3]
    elif len(st) == 3:
        outer = st
    else:
        raise SSDError(2, f"expected a 3-D or 4-D tensor, got shape {tuple(t.shape)}")
    for i, v in enumerate(outer):
        s.stride[i] = int(v)
    return s


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context under which temporaries are allocated: the stream the kernels
    run on, so that torch's caching allocator never hands a block that is still
    in use by those kernels to work on another stream."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _bad(status, msg):
    raise SSDError(status, msg)


def _check_vec(name, t, n, device, dtype=torch.float32, required=True):
    """A per-head parameter: contiguous, ``dtype``, n elements, on ``device``."""
    if t is None:
        if required:
            _bad(1, f"{name} is None")
        return
    if t.dtype != dtype:
        _bad(3, f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 1 or t.numel() != n:
        _bad(2, f"{name} must have shape ({n},), got {tuple(t.shape)}")
    if not t.is_contiguous():
        _bad(4, f"{name} must be contiguous")
    if t.device != device:
        _bad(2, f"{name} is on {t.device}, expected {device}")


def _check_state(name, t, shape, device):
    """An initial/final state or its gradient: contiguous float32 of ``shape``."""
    if t is None:
        return
    if t.dtype != torch.float32:
        _bad(3, f"{name} must be float32, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        _bad(2, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        _bad(4, f"{name} must be contiguous")
    if t.device != device:
        _bad(2, f"{name} is on {t.device}, expected {device}")


def _check_like(name, t, shape, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        _bad(2, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        _bad(2, f"{name} is on {t.device}, expected {device}")


def _check_fwd_inputs(prob, x, B, C, dt, A, dt_bias, D, z, initial_states, out=None,
                      final_states=None):
    dev = x.device
    _check_like("C", C, B.shape, dev)
    _check_like("B", B, tuple(x.shape[:-2]) + tuple(B.shape[-2:]), dev)
    _check_like("dt", dt, tuple(x.shape[:-1]), dev)
    _check_like("z", z, x.shape, dev)
    _check_like("out", out, x.shape, dev)
    H = prob.nheads
    _check_vec("A", A, H, dev)
    _check_vec("dt_bias", dt_bias, H, dev, required=False)
    _check_vec("D", D, H, dev, required=False)
    nseq = prob.nseq if prob.packed else prob.batch
    shp = (nseq, H, prob.headdim, prob.dstate)
    _check_state("initial_states", initial_states, shp, dev)
    _check_state("final_states", final_states, shp, dev)


def _workspace(need, workspace, device):
    """The caller's workspace if it is large enough, else a new one."""
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            _bad(6, "workspace must be a contiguous uint8 tensor")
        if workspace.device != device:
            _bad(6, f"workspace is on {workspace.device}, expected {device}")
        if workspace.numel() >= need:
            return workspace
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device)


@dataclass
class Problem:
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    chunk_size: int
    nseq: int = 0
    cu_seqlens: torch.Tensor | None = None     # device int32 (nseq + 1)
    chunk_meta: torch.Tensor | None = None     # device int32 table
    dt_softplus: bool = True
    dt_limit: tuple | None = None
    state_dtype: torch.dtype = torch.float32
    input_dt: bool = False                     # step size on the input term too

    def c(self) -> SsdProblem:
        p = SsdProblem()
        p.batch, p.seqlen, p.nheads, p.headdim = self.batch, self.seqlen, self.nheads, self.headdim
        p.ngroups, p.dstate, p.chunk_size, p.nseq = self.ngroups, self.dstate, self.chunk_size, self.nseq
        p.cu_seqlens = _ptr(self.cu_seqlens)
        p.chunk_meta = _ptr(self.chunk_meta)
        p.dt_softplus = 1 if self.dt_softplus else 0
        if self.dt_limit is None:
            p.dt_clamp, p.dt_min, p.dt_max = 0, 0.0, math.inf
        else:
            p.dt_clamp, p.dt_min, p.dt_max = 1, float(self.dt_limit[0]), float(self.dt_limit[1])
        p.state_dtype = _dtype_code(self.state_dtype)
        p.input_dt = 1 if self.input_dt else 0
        return p

    @property
    def packed(self) -> bool:
        return self.nseq > 0

    def check(self):
        _check(lib().ssd_problem_check(ctypes.byref(self.c())))

    def num_chunks(self) -> int:
        k = lib().ssd_num_chunks(ctypes.byref(self.c()))
        if k < 0:
            self.check()
        return int(k)

    def meta_len(self) -> int:
        return int(lib().ssd_varlen_meta_len(ctypes.byref(self.c())))

    def workspace_size(self, algo="staged") -> int:
        n = ctypes.c_size_t(0)
        _check(lib().ssd_workspace_size(ctypes.byref(self.c()), ALGO[algo], ctypes.byref(n)))
        return int(n.value)

    def backward_workspace_size(self, algo="staged", in_dtype=torch.bfloat16) -> int:
        """Workspace bytes of ssd_backward (staged) or, with another algo, of
        ssd_backward_ex for inputs of ``in_dtype``."""
        n = ctypes.c_size_t(0)
        if algo == "staged":
            _check(lib().ssd_backward_workspace_size(ctypes.byref(self.c()), ctypes.byref(n)))
        else:
            _check(lib().ssd_backward_ex_workspace_size(
                ctypes.byref(self.c()), ALGO[algo], BF16 if in_dtype == torch.bfloat16 else F32,
                ctypes.byref(n)))
        return int(n.value)


def problem_from(x, B, chunk_size, cu_seqlens=None, **kw) -> Problem:
    """Problem of x (b, T, H, P) and B (b, T, G, N), or x (T, H, P) when packed."""
    if cu_seqlens is not None:
        T, H, P = x.shape
        G, N = B.shape[1], B.shape[2]
        return Problem(1, T, H, P, G, N, chunk_size, nseq=cu_seqlens.numel() - 1,
                       cu_seqlens=cu_seqlens, **kw)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return Problem(b, T, H, P, G, N, chunk_size, **kw)


# ------------------------------------------------------------------ calls

def ssd_varlen_chunk_meta(prob: Problem, meta: torch.Tensor | None = None, stream=None):
    """Build the packed-mode chunk table on the device; returns the int32 tensor."""
    if meta is None:
        meta = torch.empty(prob.meta_len(), dtype=torch.int32, device=prob.cu_seqlens.device)
    _check(lib().ssd_varlen_chunk_meta(ctypes.byref(prob.c()), meta.data_ptr(), _stream(stream)))
    return meta


def ssd_varlen_chunk_meta_host(prob: Problem, cu_host) -> list:
    """Host twin of the chunk table (validates cu_seqlens); returns a list of ints."""
    n = prob.meta_len()
    cu = (ctypes.c_int32 * len(cu_host))(*[int(v) for v in cu_host])
    out = (ctypes.c_int32 * n)()
    _check(lib().ssd_varlen_chunk_meta_host(ctypes.byref(prob.c()), cu, out, n))
    return list(out)


def ssd_chunk_cumsum(prob: Problem, dt, A, dt_bias=None, dA_cumsum=None, dt_out=None,
                     stream=None):
    K = prob.num_chunks()
    if dA_cumsum is None:
        dA_cumsum = torch.empty((K, prob.nheads, prob.chunk_size), dtype=torch.float32,
                                device=dt.device)
    _check(lib().ssd_chunk_cumsum(ctypes.byref(prob.c()), tensor_arg(dt, packed=prob.packed),
                                  A.data_ptr(), _ptr(dt_bias), dA_cumsum.data_ptr(),
                                  _ptr(dt_out), _stream(stream)))
    return dA_cumsum


def ssd_bmm_chunk(prob: Problem, C, B, CB=None, stream=None):
    K = prob.num_chunks()
    if CB is None:
        CB = torch.empty((K, prob.ngroups, prob.chunk_size, prob.chunk_size),
                         dtype=torch.float32, device=C.device)
    _check(lib().ssd_bmm_chunk(ctypes.byref(prob.c()), tensor_arg(C, prob.packed),
                               tensor_arg(B, prob.packed), CB.data_ptr(), _stream(stream)))
    return CB


def ssd_chunk_state(prob: Problem, x, B, dA_cumsum, states=None, dt_chunk=None, stream=None):
    """dt_chunk: ssd_chunk_cumsum's dt_out, required when prob.input_dt."""
    K = prob.num_chunks()
    if states is None:
        states = torch.empty((K, prob.nheads, prob.headdim, prob.dstate),
                             dtype=prob.state_dtype, device=x.device)
    _check(lib().ssd_chunk_state(ctypes.byref(prob.c()), tensor_arg(x, prob.packed),
                                 tensor_arg(B, prob.packed), dA_cumsum.data_ptr(),
                                 _ptr(dt_chunk), states.data_ptr(), _stream(stream)))
    return states


def ssd_state_passing(prob: Problem, states, dA_cumsum, initial_states=None, states_out=None,
                      final_states=None, stream=None):
    if states_out is None:
        states_out = torch.empty_like(states)
    if final_states is None:
        nseq = prob.nseq if prob.packed else prob.batch
        final_states = torch.empty((nseq, prob.nheads, prob.headdim, prob.dstate),
                                   dtype=torch.float32, device=states.device)
    _check(lib().ssd_state_passing(ctypes.byref(prob.c()), states.data_ptr(),
                                   dA_cumsum.data_ptr(), _ptr(initial_states),
                                   states_out.data_ptr(), _ptr(final_states), _stream(stream)))
    return states_out, final_states


def ssd_chunk_scan(prob: Problem, CB, x, C, dA_cumsum, states_in, D=None, z=None, out=None,
                   out_dtype=None, dt_chunk=None, stream=None):
    """dt_chunk: ssd_chunk_cumsum's dt_out, required when prob.input_dt."""
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _check(lib().ssd_chunk_scan(ctypes.byref(prob.c()), CB.data_ptr(),
                                tensor_arg(x, prob.packed), tensor_arg(C, prob.packed),
                                dA_cumsum.data_ptr(), _ptr(dt_chunk), states_in.data_ptr(),
                                _ptr(D),
                                tensor_arg(z, prob.packed), tensor_arg(out, prob.packed),
                                _stream(stream)))
    return out


def _fwd_args(prob, x, B, C, dt, A, dt_bias, D, z, initial_states, out, final_states):
    a = SsdFwdArgs()
    pk = prob.packed
    a.x, a.B, a.C = tensor_arg(x, pk), tensor_arg(B, pk), tensor_arg(C, pk)
    a.dt = tensor_arg(dt, pk)
    a.A, a.dt_bias, a.D = A.data_ptr(), _ptr(dt_bias), _ptr(D)
    a.z = tensor_arg(z, pk)
    a.initial_states = _ptr(initial_states)
    a.out = tensor_arg(out, pk)
    a.final_states = _ptr(final_states)
    return a


def _forward_setup(x, B, C, dt, A, dt_bias, D, z, initial_states, cu_seqlens, chunk_size,
                   dt_softplus, dt_limit, state_dtype, out, out_dtype, final_states, algo,
                   workspace, stream, input_dt):
    prob = problem_from(x, B, chunk_size, cu_seqlens=cu_seqlens, dt_softplus=dt_softplus,
                        dt_limit=dt_limit, state_dtype=state_dtype, input_dt=input_dt)
    _check_fwd_inputs(prob, x, B, C, dt, A, dt_bias, D, z, initial_states, out, final_states)
    with _on(stream):
        if out is None:
            out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
        if final_states is None:
            nseq = prob.nseq if prob.packed else prob.batch
            final_states = torch.empty((nseq, prob.nheads, prob.headdim, prob.dstate),
                                       dtype=torch.float32, device=x.device)
        workspace = _workspace(prob.workspace_size(algo), workspace, x.device)
    a = _fwd_args(prob, x, B, C, dt, A, dt_bias, D, z, initial_states, out, final_states)
    return prob, a, out, final_states, workspace


def ssd_forward(x, B, C, dt, A, dt_bias=None, D=None, z=None, initial_states=None,
                cu_seqlens=None, chunk_size=128, dt_softplus=True, dt_limit=None,
                state_dtype=torch.float32, out=None, out_dtype=None, final_states=None,
                algo="staged", workspace=None, stream=None, input_dt=False):
    """The whole forward pass; returns (out, final_states).

    Batch mode: x (b, T, H, P), B and C (b, T, G, N), dt (b, T, H), z like x,
    initial_states (b, H, P, N) float32.  Packed mode: the same without the batch
    axis plus ``cu_seqlens`` (device int32, nseq + 1).  ``input_dt`` puts the
    step size on the input term as well (delta x (outer) B).  Temporaries are
    allocated on ``stream`` (the kernels' stream).
    """
    prob, a, out, final_states, workspace = _forward_setup(
        x, B, C, dt, A, dt_bias, D, z, initial_states, cu_seqlens, chunk_size, dt_softplus,
        dt_limit, state_dtype, out, out_dtype, final_states, algo, workspace, stream, input_dt)
    _check(lib().ssd_forward(ctypes.byref(prob.c()), ALGO[algo], ctypes.byref(a),
                             workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out, final_states


def ssd_forward_gated_norm(x, B, C, dt, A, weight, group_size, dt_bias=None, D=None, z=None,
                           initial_states=None, cu_seqlens=None, eps=1e-5, dt_softplus=True,
                           dt_limit=None, out=None, out_dtype=None, final_states=None,
                           rstd=None, workspace=None, stream=None, input_dt=False):
    """The fused forward with the gated RMSNorm in its epilogue
    (ssd_forward_gated_norm): out = RMSNorm_group(y silu(z)) * weight.  Returns
    (out, final_states)."""
    prob = problem_from(x, B, 128, cu_seqlens=cu_seqlens, dt_softplus=dt_softplus,
                        dt_limit=dt_limit, input_dt=input_dt)
    _check_fwd_inputs(prob, x, B, C, dt, A, dt_bias, D, z, initial_states, out, final_states)
    _check_vec("weight", weight, prob.nheads * prob.headdim, x.device)
    n = SsdNormArgs()
    n.weight, n.group_size, n.eps, n.rstd = weight.data_ptr(), int(group_size), float(eps), _ptr(rstd)
    need = ctypes.c_size_t(0)
    _check(lib().ssd_forward_gated_norm_workspace_size(ctypes.byref(prob.c()), ctypes.byref(n),
                                                       ctypes.byref(need)))
    with _on(stream):
        if out is None:
            out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
        if final_states is None:
            nseq = prob.nseq if prob.packed else prob.batch
            final_states = torch.empty((nseq, prob.nheads, prob.headdim, prob.dstate),
                                       dtype=torch.float32, device=x.device)
        workspace = _workspace(int(need.value), workspace, x.device)
    a = _fwd_args(prob, x, B, C, dt, A, dt_bias, D, z, initial_states, out, final_states)
    _check(lib().ssd_forward_gated_norm(ctypes.byref(prob.c()), ctypes.byref(a), ctypes.byref(n),
                                        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out, final_states


def ssd_forward_fused_static(x, B, C, dt, A, dt_bias=None, D=None, z=None,
                             initial_states=None, cu_seqlens=None, dt_softplus=True,
                             dt_limit=None, out=None, out_dtype=None, final_states=None,
                             stream=None, input_dt=False):
    """The fused forward with the library's static scratch array
    (ssd_forward_fused_static): no workspace is allocated.  With ``out`` and
    ``final_states`` given, nothing is allocated at all.  Returns (out,
    final_states)."""
    prob = problem_from(x, B, 128, cu_seqlens=cu_seqlens, dt_softplus=dt_softplus,
                        dt_limit=dt_limit, input_dt=input_dt)
    _check_fwd_inputs(prob, x, B, C, dt, A, dt_bias, D, z, initial_states, out, final_states)
    with _on(stream):
        if out is None:
            out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
        if final_states is None:
            nseq = prob.nseq if prob.packed else prob.batch
            final_states = torch.empty((nseq, prob.nheads, prob.headdim, prob.dstate),
                                       dtype=torch.float32, device=x.device)
    a = _fwd_args(prob, x, B, C, dt, A, dt_bias, D, z, initial_states, out, final_states)
    _check(lib().ssd_forward_fused_static(ctypes.byref(prob.c()), ctypes.byref(a),
                                          _stream(stream)))
    return out, final_states


@dataclass
class Grads:
    dx: torch.Tensor
    dB: torch.Tensor
    dC: torch.Tensor
    ddt: torch.Tensor
    dA: torch.Tensor
    ddt_bias: torch.Tensor
    dD: torch.Tensor | None
    dz: torch.Tensor | None
    dinitial_states: torch.Tensor


def _bwd_alloc(prob, x, B, C, dt, D, z, nseq, workspace, algo):
    dev, f32 = x.device, torch.float32
    g = Grads(dx=torch.empty(x.shape, dtype=f32, device=dev),
              dB=torch.empty(B.shape, dtype=f32, device=dev),
              dC=torch.empty(C.shape, dtype=f32, device=dev),
              ddt=torch.empty(dt.shape, dtype=f32, device=dev),
              dA=torch.empty(prob.nheads, dtype=f32, device=dev),
              ddt_bias=torch.empty(prob.nheads, dtype=f32, device=dev),
              dD=torch.empty(prob.nheads, dtype=f32, device=dev) if D is not None else None,
              dz=torch.empty(x.shape, dtype=f32, device=dev) if z is not None else None,
              dinitial_states=torch.empty((nseq, prob.nheads, prob.headdim, prob.dstate),
                                          dtype=f32, device=dev))
    if workspace is not None and algo != "staged":
        # the per-chunk backward takes any workspace down to its smallest head
        # pass (fewer heads per pass in a smaller one); the library checks it
        _workspace(0, workspace, dev)
        return g, workspace
    return g, _workspace(prob.backward_workspace_size(algo, x.dtype), workspace, dev)


def ssd_backward(x, B, C, dt, A, dout, dt_bias=None, D=None, z=None, initial_states=None,
                 dfinal_states=None, cu_seqlens=None, chunk_size=128, dt_softplus=True,
                 dt_limit=None, workspace=None, stream=None, input_dt=False,
                 algo="auto") -> Grads:
    """Gradients of sum(dout * out) + sum(dfinal_states * final_states) with
    respect to every input of ``ssd_forward`` (same arguments and layouts);
    all gradients are float32, allocated on ``stream`` like the workspace.
    ``algo``: "staged" (ssd_backward), "fused" (the per-chunk backward of
    ssd_backward_ex) or "auto" (fused where it applies).  A ``workspace``
    given for "fused" or "auto" is used as it is: one smaller than
    ``Problem.backward_workspace_size`` makes the per-chunk backward take its
    heads in more passes (down to one group, or eight heads of a group)."""
    prob = problem_from(x, B, chunk_size, cu_seqlens=cu_seqlens, dt_softplus=dt_softplus,
                        dt_limit=dt_limit, input_dt=input_dt)
    _check_fwd_inputs(prob, x, B, C, dt, A, dt_bias, D, z, initial_states)
    _check_like("dout", dout, x.shape, x.device)
    nseq = prob.nseq if prob.packed else prob.batch
    _check_state("dfinal_states", dfinal_states, (nseq, prob.nheads, prob.headdim, prob.dstate),
                 x.device)
    with _on(stream):
        g, workspace = _bwd_alloc(prob, x, B, C, dt, D, z, nseq, workspace, algo)
    a = SsdBwdArgs()
    pk = prob.packed
    a.x, a.B, a.C = tensor_arg(x, pk), tensor_arg(B, pk), tensor_arg(C, pk)
    a.dt = tensor_arg(dt, pk)
    a.A, a.dt_bias, a.D = A.data_ptr(), _ptr(dt_bias), _ptr(D)
    a.z = tensor_arg(z, pk)
    a.initial_states = _ptr(initial_states)
    a.dout = tensor_arg(dout, pk)
    a.dfinal_states = _ptr(dfinal_states)
    a.dx, a.dB, a.dC = tensor_arg(g.dx, pk), tensor_arg(g.dB, pk), tensor_arg(g.dC, pk)
    a.ddt, a.dz = tensor_arg(g.ddt, pk), tensor_arg(g.dz, pk)
    a.dA, a.ddt_bias, a.dD = g.dA.data_ptr(), g.ddt_bias.data_ptr(), _ptr(g.dD)
    a.dinitial_states = g.dinitial_states.data_ptr()
    if algo == "staged":
        _check(lib().ssd_backward(ctypes.byref(prob.c()), ctypes.byref(a), workspace.data_ptr(),
                                  workspace.numel(), _stream(stream)))
    else:
        _check(lib().ssd_backward_ex(ctypes.byref(prob.c()), ctypes.byref(a), ALGO[algo],
                                     workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return g


# ------------------------------------------------------------------ complex A

def _cx_tensor(t: torch.Tensor | None, packed: bool = False) -> SsdTensor:
    """ssd_tensor of a complex64 (b, T, H, X) tensor, or (T, H, X) when packed:
    float32 pairs, strides in complex elements (the innermost must be 1)."""
    s = SsdTensor()
    s.dtype = F32
    if t is None or t.numel() == 0:
        s.data = None
        return s
    if t.dtype != torch.complex64:
        raise SSDError(3, f"expected complex64, got {t.dtype}")
    want = 3 if packed else 4
    if t.dim() != want:
        raise SSDError(2, f"expected a {want}-D tensor, got shape {tuple(t.shape)}")
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise SSDError(4, "innermost dimension must be contiguous")
    s.data = t.data_ptr()
    st = ([0] if packed else []) + [int(v) for v in t.stride()]
    for i in range(3):
        s.stride[i] = st[i]
    return s


@dataclass
class ComplexProblem:
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    chunk_size: int = 64
    nseq: int = 0
    cu_seqlens: torch.Tensor | None = None   # device int32 (nseq + 1), packed mode

    def c(self) -> SsdComplexProblem:
        p = SsdComplexProblem()
        p.batch, p.seqlen, p.nheads = self.batch, self.seqlen, self.nheads
        p.headdim, p.dstate, p.chunk_size = self.headdim, self.dstate, self.chunk_size
        p.nseq = self.nseq
        p.cu_seqlens = _ptr(self.cu_seqlens)
        return p

    def check(self):
        _check(lib().ssd_complex_problem_check(ctypes.byref(self.c())))

    def workspace_size(self) -> int:
        n = ctypes.c_size_t(0)
        _check(lib().ssd_complex_workspace_size(ctypes.byref(self.c()), ctypes.byref(n)))
        return int(n.value)


def ssd_complex_forward(x, B, C, dt, A, initial_states=None, chunk_size=64,
                        out_complex=False, out=None, final_states=None, workspace=None,
                        cu_seqlens=None, stream=None):
    """The complex-A SSD forward (ssd_complex_forward).

    x (b, T, H, P), B and C (b, T, H, N) complex64; dt (b, T, H) float32; A (H,)
    complex64; initial_states (b, H, P, N) complex64 or None.  Packed mode
    (cu_seqlens: device int32, nseq + 1 offsets): the token tensors have no batch
    axis and the states are per sequence.  Returns (out, final_states): out is
    float32 (the real part) or, with out_complex, complex64.
    """
    packed = cu_seqlens is not None
    if packed:
        T, H, P = x.shape
        N = B.shape[2]
        nseq = cu_seqlens.numel() - 1
        prob = ComplexProblem(1, T, H, P, N, chunk_size, nseq=nseq, cu_seqlens=cu_seqlens)
        lead, ns = (T,), nseq
    else:
        b, T, H, P = x.shape
        N = B.shape[3]
        prob = ComplexProblem(b, T, H, P, N, chunk_size)
        lead, ns = (b, T), b
    dev = x.device
    _check_like("B", B, lead + (H, N), dev)
    _check_like("C", C, lead + (H, N), dev)
    _check_like("dt", dt, lead + (H,), dev)
    _check_vec("A", A, H, dev, dtype=torch.complex64)
    if dt.dtype != torch.float32:
        raise SSDError(3, "dt must be float32")
    for name, t in (("initial_states", initial_states), ("final_states", final_states)):
        if t is None:
            continue
        if t.dtype != torch.complex64 or tuple(t.shape) != (ns, H, P, N):
            raise SSDError(2, f"{name} must be complex64 of shape {(ns, H, P, N)}")
        if not t.is_contiguous():
            raise SSDError(4, f"{name} must be contiguous")
    with _on(stream):
        if out is None:
            out = torch.empty(lead + (H, P),
                              dtype=torch.complex64 if out_complex else torch.float32,
                              device=dev)
        if final_states is None:
            final_states = torch.empty((ns, H, P, N), dtype=torch.complex64, device=dev)
        workspace = _workspace(prob.workspace_size(), workspace, dev)
    a = SsdComplexFwdArgs()
    a.x, a.B, a.C = (_cx_tensor(x, packed), _cx_tensor(B, packed), _cx_tensor(C, packed))
    a.dt = tensor_arg(dt, packed)
    a.A = A.data_ptr()
    a.initial_states = _ptr(initial_states)
    if out_complex:
        a.out = _cx_tensor(out, packed)
    else:
        a.out = tensor_arg(out, packed)
    a.out_complex = 1 if out_complex else 0
    a.final_states = final_states.data_ptr()
    _check(lib().ssd_complex_forward(ctypes.byref(prob.c()), ctypes.byref(a),
                                     workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out, final_states


def ssd_complex_chunk_state(prob: ComplexProblem, x, B, dt, A, states, chunk_dt_sum,
                            stream=None):
    """Every chunk's end state from a zero start; states (b * nc, H, P, N)
    complex64, chunk_dt_sum (b, H, nc) float32, both written."""
    _check(lib().ssd_complex_chunk_state(ctypes.byref(prob.c()), _cx_tensor(x), _cx_tensor(B),
                                         tensor_arg(dt), A.data_ptr(), _ptr(states),
                                         _ptr(chunk_dt_sum), _stream(stream)))
    return states, chunk_dt_sum


def ssd_complex_state_passing(prob: ComplexProblem, A, chunk_dt_sum, states,
                              initial_states=None, final_states=None, stream=None):
    """In place: chunk states -> carry-in states; also the final states."""
    _check(lib().ssd_complex_state_passing(ctypes.byref(prob.c()), A.data_ptr(),
                                           _ptr(chunk_dt_sum), _ptr(initial_states),
                                           _ptr(states), _ptr(final_states), _stream(stream)))
    return states, final_states


def ssd_complex_chunk_scan(prob: ComplexProblem, x, B, C, dt, A, states_in, out,
                           stream=None):
    """The output from the carry-in states; out float32 (real part) or complex64."""
    oc = out.dtype == torch.complex64
    _check(lib().ssd_complex_chunk_scan(ctypes.byref(prob.c()), _cx_tensor(x), _cx_tensor(B),
                                        _cx_tensor(C), tensor_arg(dt), A.data_ptr(),
                                        _ptr(states_in), _cx_tensor(out) if oc else tensor_arg(out),
                                        1 if oc else 0, _stream(stream)))
    return out


# ------------------------------------------------------------------ gated RMSNorm

def norm_problem(y, group_size, eps=1e-5) -> SsdNormProblem:
    b, T, H, P = y.shape
    p = SsdNormProblem()
    p.batch, p.seqlen, p.nheads, p.headdim = b, T, H, P
    p.group_size, p.eps = int(group_size), float(eps)
    return p


def ssd_gated_rmsnorm_fwd(y, z, weight, group_size, eps=1e-5, out=None, out_dtype=None,
                          rstd=None, stream=None):
    """out = g / sqrt(mean_group(g^2) + eps) * weight, g = y silu(z); y, z (b, T, H, P).
    Returns (out, rstd); rstd is written only when a tensor is passed."""
    _check_like("z", z, y.shape, y.device)
    _check_like("out", out, y.shape, y.device)
    _check_vec("weight", weight, y.shape[2] * y.shape[3], y.device)
    with _on(stream):
        if out is None:
            out = torch.empty(y.shape, dtype=out_dtype or y.dtype, device=y.device)
    p = norm_problem(y, group_size, eps)
    _check(lib().ssd_gated_rmsnorm_fwd(ctypes.byref(p), tensor_arg(y), tensor_arg(z),
                                       weight.data_ptr(), tensor_arg(out), _ptr(rstd),
                                       _stream(stream)))
    return out, rstd


def gated_rmsnorm_bwd_workspace_size(y, group_size, eps=1e-5) -> int:
    p = norm_problem(y, group_size, eps)
    n = ctypes.c_size_t(0)
    _check(lib().ssd_gated_rmsnorm_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def ssd_gated_rmsnorm_bwd(y, z, weight, dout, group_size, eps=1e-5, workspace=None,
                          dy=None, dz=None, dw=None, stream=None):
    """Gradients (dy, dz, dweight) of sum(dout * out); float32.  Output tensors and
    the workspace are allocated when not given."""
    p = norm_problem(y, group_size, eps)
    _check_like("z", z, y.shape, y.device)
    _check_like("dout", dout, y.shape, y.device)
    _check_vec("weight", weight, y.shape[2] * y.shape[3], y.device)
    with _on(stream):
        workspace = _workspace(gated_rmsnorm_bwd_workspace_size(y, group_size, eps), workspace,
                               y.device)
        if dy is None:
            dy = torch.empty(y.shape, dtype=torch.float32, device=y.device)
        if dz is None and z is not None:
            dz = torch.empty(y.shape, dtype=torch.float32, device=y.device)
        if dw is None:
            dw = torch.empty(weight.shape, dtype=torch.float32, device=y.device)
    _check(lib().ssd_gated_rmsnorm_bwd(ctypes.byref(p), tensor_arg(y), tensor_arg(z),
                                       weight.data_ptr(), tensor_arg(dout), tensor_arg(dy),
                                       tensor_arg(dz), dw.data_ptr(), workspace.data_ptr(),
                                       workspace.numel(), _stream(stream)))
    return dy, dz, dw
