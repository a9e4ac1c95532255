"""The C ABI on the host: loads, exports every declared symbol, validates.

No GPU is needed: every call here either is host-only (problem checks, sizes,
the host chunk table) or fails validation before anything is launched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from mamba_ssd_chunked_scan_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(ssd_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_stage_calls():
    names = declared_functions()
    for n in ("ssd_chunk_cumsum", "ssd_bmm_chunk", "ssd_chunk_state", "ssd_state_passing",
              "ssd_chunk_scan", "ssd_forward", "ssd_varlen_chunk_meta"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ssd.lib()
    names = declared_functions()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, f"declared but not exported: {missing}"
    assert set(ssd.EXPORTS) == set(names)


def test_version_and_status_strings():
    L = ssd.lib()
    assert b"gfx950" in L.ssd_version()
    for code, name in ssd.STATUS.items():
        assert L.ssd_status_string(code).decode() == name


def prob(**kw):
    base = dict(batch=1, seqlen=8192, nheads=64, headdim=64, ngroups=8, dstate=128,
                chunk_size=128)
    base.update(kw)
    return ssd.Problem(**base)


def status_of(p):
    return ssd.lib().ssd_problem_check(ctypes.byref(p.c()))


@pytest.mark.parametrize("kw,code,word", [
    (dict(headdim=60), 5, "headdim"),
    (dict(headdim=512), 5, "headdim"),
    (dict(dstate=8), 5, "dstate"),
    (dict(chunk_size=100), 5, "chunk_size"),
    (dict(nheads=6, ngroups=4), 2, "ngroups"),
    (dict(batch=0), 2, "batch"),
    (dict(seqlen=-1), 2, "seqlen"),
    (dict(batch=2, nseq=3), 2, "packed"),
    (dict(nseq=3), 1, "cu_seqlens"),
    (dict(dt_limit=(0.5, 0.1)), 2, "dt_min"),
])
def test_problem_check_rejects(kw, code, word):
    p = prob(**kw)
    if kw.get("nseq") and kw.get("batch", 1) == 1:
        p.cu_seqlens = None
    assert status_of(p) == code
    assert word in ssd.lib().ssd_last_error_message().decode()


def test_problem_check_accepts_all_workload_shapes():
    for kw in (dict(), dict(nheads=128, ngroups=1), dict(seqlen=65536, nheads=80, ngroups=1,
                                                         chunk_size=256),
               dict(seqlen=256, nheads=4, headdim=16, ngroups=1, dstate=16, chunk_size=64),
               dict(nheads=6, ngroups=2), dict(seqlen=0)):
        assert status_of(prob(**kw)) == 0


def test_num_chunks_and_sizes():
    assert prob().num_chunks() == 64
    assert prob(batch=3, seqlen=1000).num_chunks() == 3 * 8
    assert prob(seqlen=0).num_chunks() == 0
    p = prob(nseq=8)
    p.cu_seqlens = None
    c = p.c()
    c.cu_seqlens = 1  # any non-NULL value: nothing is dereferenced on the host
    L = ssd.lib()
    assert L.ssd_num_chunks(ctypes.byref(c)) == 64 + 8
    assert L.ssd_varlen_meta_len(ctypes.byref(c)) == 4 + 3 * 72 + 9
    n = ctypes.c_size_t()
    assert L.ssd_workspace_size(ctypes.byref(prob().c()), 0, ctypes.byref(n)) == 0
    K, H, C, G, P, N = 64, 64, 128, 8, 64, 128
    assert n.value == K * H * C * 4 + K * G * C * C * 4 + K * H * P * N * 4


def fake_tensor(addr=4096, dtype=ssd.BF16, strides=(8192 * 6144, 6144, 64)):
    t = ssd.SsdTensor()
    t.data = addr
    t.dtype = dtype
    for i, s in enumerate(strides):
        t.stride[i] = s
    return t


def test_tensor_validation_before_launch():
    # Every case fails on the host; the pointers are never dereferenced.
    L = ssd.lib()
    p = prob().c()
    good = fake_tensor()
    null = ssd.SsdTensor()
    cases = [
        (null, good, 1),                                   # C missing
        (fake_tensor(addr=4098), good, 4),                 # misaligned base
        (fake_tensor(strides=(0, 6143, 64)), good, 4),     # row stride breaks alignment
        (fake_tensor(strides=(0, -6144, 64)), good, 4),    # negative stride
        (fake_tensor(dtype=7), good, 3),                   # unknown dtype
        (good, fake_tensor(dtype=ssd.F32), 3),             # B and C dtypes differ
    ]
    for Ct, Bt, code in cases:
        rc = L.ssd_bmm_chunk(ctypes.byref(p), Ct, Bt, 4096, None)
        assert rc == code, (rc, code, L.ssd_last_error_message())
    assert L.ssd_bmm_chunk(ctypes.byref(p), good, good, None, None) == 1


def test_forward_validation_workspace_and_algo():
    L = ssd.lib()
    p = prob().c()
    a = ssd.SsdFwdArgs()
    a.x = fake_tensor(strides=(8192 * 4096, 4096, 64))
    a.B = fake_tensor()
    a.C = fake_tensor()
    a.dt = fake_tensor(strides=(8192 * 64, 64, 1))
    a.out = fake_tensor(strides=(8192 * 4096, 4096, 64))
    a.A = 4096
    assert L.ssd_forward(ctypes.byref(p), 0, ctypes.byref(a), None, 0, None) == 6
    assert L.ssd_forward(ctypes.byref(p), 0, ctypes.byref(a), 4096, 100, None) == 6
    assert b"need" in L.ssd_last_error_message()
    assert L.ssd_forward(ctypes.byref(p), 9, ctypes.byref(a), 4096, 1 << 40, None) == 5
    a.A = None
    assert L.ssd_forward(ctypes.byref(p), 0, ctypes.byref(a), 4096, 1 << 40, None) == 1


def test_fused_paths_refuse_token_strides_past_32_bit_offsets():
    # The fused forward and the per-chunk backward address a 128-token chunk's
    # rows as 32-bit byte offsets; a token stride of 2^24 bf16 elements puts 127
    # rows 4 GiB apart, so both refuse it on the host (nothing is launched).
    L = ssd.lib()
    p = prob().c()
    huge = (0, 1 << 24, 64)
    a = ssd.SsdFwdArgs()
    a.x = fake_tensor(strides=huge)
    a.B = fake_tensor()
    a.C = fake_tensor()
    a.dt = fake_tensor(strides=(8192 * 64, 64, 1))
    a.out = fake_tensor(strides=(8192 * 4096, 4096, 64))
    a.A = 4096
    rc = L.ssd_forward(ctypes.byref(p), ssd.ALGO["fused"], ctypes.byref(a), 4096, 1 << 40, None)
    assert rc == 5 and b"2 GiB" in L.ssd_last_error_message(), (rc, L.ssd_last_error_message())
    b = ssd.SsdBwdArgs()
    tok, grp, steps = (8192 * 4096, 4096, 64), (8192 * 1024, 1024, 128), (8192 * 64, 64, 1)
    b.x = fake_tensor(strides=huge)
    b.B, b.C = fake_tensor(strides=grp), fake_tensor(strides=grp)
    b.dt = fake_tensor(strides=steps)
    b.dout = fake_tensor(dtype=ssd.F32, strides=tok)
    b.dx = fake_tensor(dtype=ssd.F32, strides=tok)
    b.dB, b.dC = fake_tensor(dtype=ssd.F32, strides=grp), fake_tensor(dtype=ssd.F32, strides=grp)
    b.ddt = fake_tensor(dtype=ssd.F32, strides=steps)
    b.A = b.dA = b.ddt_bias = 4096
    rc = L.ssd_backward_ex(ctypes.byref(p), ctypes.byref(b), ssd.ALGO["fused"], 4096, 1 << 40,
                           None)
    assert rc == 5 and b"2 GiB" in L.ssd_last_error_message(), (rc, L.ssd_last_error_message())


def test_backward_validation_before_launch():
    # fake device addresses: every case fails on the host before any launch
    L = ssd.lib()
    p = prob().c()
    tok = (8192 * 4096, 4096, 64)
    grp = (8192 * 1024, 1024, 128)
    steps = (8192 * 64, 64, 1)
    a = ssd.SsdBwdArgs()
    a.x = fake_tensor(strides=tok)
    a.B = fake_tensor(strides=grp)
    a.C = fake_tensor(strides=grp)
    a.dt = fake_tensor(strides=steps)
    a.dout = fake_tensor(dtype=ssd.F32, strides=tok)
    a.dx = fake_tensor(dtype=ssd.F32, strides=tok)
    a.dB = fake_tensor(dtype=ssd.F32, strides=grp)
    a.dC = fake_tensor(dtype=ssd.F32, strides=grp)
    a.ddt = fake_tensor(dtype=ssd.F32, strides=steps)
    a.A = a.dA = a.ddt_bias = 4096
    n = ctypes.c_size_t()
    assert L.ssd_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    big = n.value
    assert L.ssd_backward(ctypes.byref(p), ctypes.byref(a), 4096, big - 1, None) == 6
    assert b"need" in L.ssd_last_error_message()
    assert L.ssd_backward(ctypes.byref(p), ctypes.byref(a), 4096 + 16, big, None) == 6
    for name in ("initial_states", "dfinal_states", "dinitial_states"):
        setattr(a, name, 4096 + 4)
        assert L.ssd_backward(ctypes.byref(p), ctypes.byref(a), 4096, big, None) == 4, name
        assert name.encode() in L.ssd_last_error_message()
        setattr(a, name, None)
    a.z = fake_tensor(strides=tok)  # a gate needs dz
    assert L.ssd_backward(ctypes.byref(p), ctypes.byref(a), 4096, big, None) == 1
    a.z = ssd.SsdTensor()
    a.ddt = fake_tensor(strides=steps)  # ddt must be fp32
    assert L.ssd_backward(ctypes.byref(p), ctypes.byref(a), 4096, big, None) == 3
    a.ddt = fake_tensor(dtype=ssd.F32, strides=steps)
    a.dA = None
    assert L.ssd_backward(ctypes.byref(p), ctypes.byref(a), 4096, big, None) == 1


def host_meta(cu, C):
    T = int(cu[-1])
    p = ssd.Problem(1, T, 4, 16, 1, 16, C, nseq=len(cu) - 1)
    c = p.c()
    c.cu_seqlens = 1
    L = ssd.lib()
    n = L.ssd_varlen_meta_len(ctypes.byref(c))
    arr = (ctypes.c_int32 * len(cu))(*[int(v) for v in cu])
    out = (ctypes.c_int32 * n)()
    rc = L.ssd_varlen_chunk_meta_host(ctypes.byref(c), arr, out, n)
    return rc, list(out)


def expected_table(cu, C):
    m = oracle.varlen_chunk_meta(cu, C)
    T, nseq = int(cu[-1]), len(cu) - 1
    K = -(-T // C) + nseq
    tab = [m.nchunks, nseq, C, K]
    for j in range(K):
        tab += [m.seq[j], m.start[j], m.length[j]] if j < m.nchunks else [-1, 0, 0]
    return tab + m.first_chunk


def test_host_chunk_table_matches_oracle_bit_exact():
    rng = np.random.default_rng(1)
    C = 32
    for lens in ([1], [32], [33], [0, 5], [31, 32, 33, 0, 64, 65], [0, 0, 7], [100, 0]):
        cu = [0] + list(np.cumsum(lens))
        rc, tab = host_meta(cu, C)
        assert rc == 0
        assert tab == expected_table(cu, C)
    for _ in range(100):
        nseq = int(rng.integers(1, 12))
        T = int(rng.integers(1, 3000))
        cuts = np.sort(rng.integers(0, T + 1, nseq - 1))
        cu = [0] + [int(v) for v in cuts] + [T]
        Cc = int(rng.choice([32, 64, 128, 256]))
        rc, tab = host_meta(cu, Cc)
        assert rc == 0 and tab == expected_table(cu, Cc)


def test_host_chunk_table_rejects_bad_cu_seqlens():
    for cu in ([1, 5, 9], [0, 5, 3, 9], [0, 4, 8]):
        p = ssd.Problem(1, 9, 4, 16, 1, 16, 32, nseq=len(cu) - 1)
        c = p.c()
        c.cu_seqlens = 1
        L = ssd.lib()
        n = L.ssd_varlen_meta_len(ctypes.byref(c))
        arr = (ctypes.c_int32 * len(cu))(*cu)
        out = (ctypes.c_int32 * n)()
        assert L.ssd_varlen_chunk_meta_host(ctypes.byref(c), arr, out, n) == 2


# ------------------------------------------------------------------ complex A

def cx_prob(**kw):
    base = dict(batch=8, seqlen=2048, nheads=16, headdim=64, dstate=64, chunk_size=64)
    base.update(kw)
    return ssd.ComplexProblem(**base)


@pytest.mark.parametrize("kw,code,word", [
    (dict(headdim=144), 5, "headdim"),
    (dict(headdim=40), 5, "headdim"),
    (dict(dstate=24), 5, "dstate"),
    (dict(chunk_size=48), 5, "chunk_size"),
    (dict(batch=0), 2, "batch"),
    (dict(seqlen=-1), 2, "seqlen"),
    (dict(nheads=0), 2, "nheads"),
    (dict(batch=5000, nheads=16), 5, "nheads"),
])
def test_complex_problem_check_names_the_dim(kw, code, word):
    L = ssd.lib()
    rc = L.ssd_complex_problem_check(ctypes.byref(cx_prob(**kw).c()))
    assert rc == code
    assert word in L.ssd_last_error_message().decode()


def test_complex_workspace_size():
    p = cx_prob()
    nc = 2048 // 64
    states = 8 * nc * 16 * 64 * 64 * 8
    lam = 8 * 16 * nc * 4
    r256 = lambda v: (v + 255) // 256 * 256
    assert p.workspace_size() == r256(states) + r256(lam)
    assert cx_prob(seqlen=0).workspace_size() == 0


def test_complex_forward_rejects_bad_arguments_before_launching():
    L = ssd.lib()
    p = cx_prob(batch=1, seqlen=64, nheads=2, headdim=16, dstate=16)
    a = ssd.SsdComplexFwdArgs()
    # x missing
    rc = L.ssd_complex_forward(ctypes.byref(p.c()), ctypes.byref(a), None, 0, None)
    assert rc == 1 and "x" in L.ssd_last_error_message().decode()
    # x of the wrong dtype
    buf = (ctypes.c_char * 4096)()
    base = (ctypes.addressof(buf) + 255) // 256 * 256
    a.x.data, a.x.dtype = base, 1
    rc = L.ssd_complex_forward(ctypes.byref(p.c()), ctypes.byref(a), None, 0, None)
    assert rc == 3 and "complex64" in L.ssd_last_error_message().decode()
    # odd stride (rows not 16-byte aligned)
    a.x.dtype = 0
    a.x.stride[0], a.x.stride[1], a.x.stride[2] = 64 * 2 * 16, 2 * 16 + 1, 16
    rc = L.ssd_complex_forward(ctypes.byref(p.c()), ctypes.byref(a), None, 0, None)
    assert rc == 4 and "stride[1]" in L.ssd_last_error_message().decode()


# ------------------------------------------------------------------ gated RMSNorm

@pytest.mark.parametrize("kw,code,word", [
    (dict(nheads=6, group_size=96), 5, "group_size"),
    (dict(group_size=1000), 2, "group_size"),
    (dict(headdim=12), 5, "headdim"),
    (dict(eps=-1.0), 2, "eps"),
    (dict(batch=0), 2, "batch"),
])
def test_norm_problem_check(kw, code, word):
    L = ssd.lib()
    p = ssd.SsdNormProblem()
    base = dict(batch=1, seqlen=16, nheads=8, headdim=64, group_size=512, eps=1e-5)
    base.update(kw)
    for k, v in base.items():
        setattr(p, k, v)
    ws = ctypes.c_size_t(0)
    rc = L.ssd_gated_rmsnorm_bwd_workspace_size(ctypes.byref(p), ctypes.byref(ws))
    assert rc == code
    assert word in L.ssd_last_error_message().decode()


def test_norm_workspace_size():
    L = ssd.lib()
    p = ssd.SsdNormProblem()
    p.batch, p.seqlen, p.nheads, p.headdim, p.group_size, p.eps = 1, 8192, 64, 64, 512, 1e-5
    ws = ctypes.c_size_t(0)
    assert L.ssd_gated_rmsnorm_bwd_workspace_size(ctypes.byref(p), ctypes.byref(ws)) == 0
    assert ws.value == 128 * 4096 * 4           # 64-token tiles x channels, no statistics
    p.group_size = 1024
    assert L.ssd_gated_rmsnorm_bwd_workspace_size(ctypes.byref(p), ctypes.byref(ws)) == 0
    assert ws.value == 128 * 4096 * 4 + 8192 * 4 * 8


def test_norm_rejects_too_many_vectors():
    L = ssd.lib()
    p = ssd.SsdNormProblem()
    p.batch, p.seqlen, p.nheads, p.headdim, p.group_size, p.eps = 64, 65536, 64, 64, 512, 1e-5
    ws = ctypes.c_size_t(0)
    assert L.ssd_gated_rmsnorm_bwd_workspace_size(ctypes.byref(p), ctypes.byref(ws)) == 5
    assert "2^31" in L.ssd_last_error_message().decode()


def test_complex_packed_checks():
    L = ssd.lib()
    p = cx_prob(batch=2, seqlen=100, nseq=3)
    assert L.ssd_complex_problem_check(ctypes.byref(p.c())) == 2
    assert "batch == 1" in L.ssd_last_error_message().decode()
    p = cx_prob(batch=1, seqlen=100, nseq=3)
    assert L.ssd_complex_problem_check(ctypes.byref(p.c())) == 1
    assert "cu_seqlens" in L.ssd_last_error_message().decode()
    # the stage calls take batch problems only
    c = p.c()
    buf = (ctypes.c_int32 * 4)(0, 10, 50, 100)
    c.cu_seqlens = ctypes.cast(buf, ctypes.c_void_p)
    rc = L.ssd_complex_chunk_state(ctypes.byref(c), ssd.SsdTensor(), ssd.SsdTensor(),
                                   ssd.SsdTensor(), None, None, None, None)
    assert rc == 5 and "ssd_complex_forward" in L.ssd_last_error_message().decode()


def test_complex_packed_workspace_includes_chunk_table():
    L = ssd.lib()
    p = cx_prob(batch=1, seqlen=1000, nseq=5, chunk_size=64)
    c = p.c()
    buf = (ctypes.c_int32 * 6)(0, 100, 200, 300, 400, 1000)
    c.cu_seqlens = ctypes.cast(buf, ctypes.c_void_p)
    ws = ctypes.c_size_t(0)
    assert L.ssd_complex_workspace_size(ctypes.byref(c), ctypes.byref(ws)) == 0
    K = 16 + 5
    r256 = lambda v: (v + 255) // 256 * 256
    assert ws.value == r256(K * 16 * 64 * 64 * 8) + r256(16 * K * 4) + r256((4 + 3 * K + 6) * 4)
