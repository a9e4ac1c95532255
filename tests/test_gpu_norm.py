"""Parity of the gated RMSNorm (ssd_gated_rmsnorm_fwd / _bwd) with the fp64 oracle.

Gates: fp32 inputs, fp32 output: max|gpu - ref| / RMS(ref) <= 1e-4 (the fp32
gate); bf16 inputs: the oracle reads the same bf16 values, fp32 output within
1e-4 as well (the pass computes in fp32 from exact inputs), bf16 output within
one bf16 rounding per element (2^-8 |ref|) plus 1e-4 RMS.  Gradients (fp32):
1e-4 of their RMS; the weight gradient sums over every token, so 1e-4 of its RMS
too.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import err
from mamba_ssd_chunked_scan_amd import ssd
from mamba_ssd_chunked_scan_amd.inputs import round_bf16

pytestmark = pytest.mark.gpu
TOL = 1e-4


def make(seed, b, T, H, P, bf16):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((b, T, H, P)).astype(np.float32) * 4.0
    z = rng.standard_normal((b, T, H, P)).astype(np.float32)
    w = (1.0 + 0.3 * rng.standard_normal(H * P)).astype(np.float32)
    dout = rng.standard_normal((b, T, H, P)).astype(np.float32)
    if bf16:
        y, z, dout = round_bf16(y), round_bf16(z), round_bf16(dout)
    return y, z, w, dout


def dev(a, dt):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)


@pytest.mark.parametrize("shape,gs", [
    ((1, 300, 8, 64), 512),      # Nemotron-Nano's group: 8 heads x 64
    ((2, 77, 4, 16), 16),        # groups inside a head
    ((1, 50, 6, 32), 64),        # groups spanning two heads
    ((1, 40, 16, 64), 1024),     # wider than a strip (statistics pass)
    ((1, 33, 12, 16), 8),
    ((1, 20, 128, 64), 8192),    # Granite's one group of d_inner = 8192 channels
])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("gated", [True, False])
def test_forward_and_backward(shape, gs, bf16, gated):
    b, T, H, P = shape
    y, z, w, dout = make(sum(shape) + gs, b, T, H, P, bf16)
    if not gated:
        z = None
    dt = torch.bfloat16 if bf16 else torch.float32
    ref = oracle.gated_rmsnorm_fwd(y, z, w, gs, eps=1e-5)
    out, _ = ssd.ssd_gated_rmsnorm_fwd(dev(y, dt), dev(z, dt), dev(w, torch.float32), gs,
                                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    e = err(out.cpu().numpy(), ref.out)
    assert e <= TOL, e
    g = oracle.gated_rmsnorm_bwd(y, z, w, dout, gs, eps=1e-5)
    dy, dz, dw = ssd.ssd_gated_rmsnorm_bwd(dev(y, dt), dev(z, dt), dev(w, torch.float32),
                                           dev(dout, dt), gs)
    torch.cuda.synchronize()
    e_dy = err(dy.cpu().numpy(), g.dy)
    e_dw = err(dw.cpu().numpy(), g.dweight)
    print(f"norm {shape} gs {gs}: out {e:.2e} dy {e_dy:.2e} dw {e_dw:.2e}")
    assert e_dy <= TOL and e_dw <= TOL, (e_dy, e_dw)
    if gated:
        e_dz = err(dz.cpu().numpy(), g.dz)
        assert e_dz <= TOL, e_dz


def test_bf16_output_and_rstd():
    y, z, w, _ = make(3, 1, 64, 8, 64, True)
    ref = oracle.gated_rmsnorm_fwd(y, z, w, 512, eps=1e-5)
    rstd = torch.empty((64, 1), dtype=torch.float32, device="cuda")
    out, _ = ssd.ssd_gated_rmsnorm_fwd(dev(y, torch.bfloat16), dev(z, torch.bfloat16),
                                       dev(w, torch.float32), 512, rstd=rstd)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref.out ** 2))
    assert np.all(np.abs(o - ref.out) <= TOL * rms + 2.0 ** -8 * np.abs(ref.out))
    assert err(rstd.cpu().numpy().reshape(-1), ref.rstd.reshape(-1)) <= 1e-5


def test_strided_views_and_determinism():
    # y as the x-part of a packed buffer; two backward runs bit-identical
    y, z, w, dout = make(5, 2, 100, 4, 32, False)
    packed = np.concatenate([y, np.zeros((2, 100, 4, 16), np.float32)], axis=-1)
    t = dev(packed, torch.float32)
    yv = t[..., :32]
    ref = oracle.gated_rmsnorm_fwd(y, z, w, 64, eps=1e-5)
    out, _ = ssd.ssd_gated_rmsnorm_fwd(yv, dev(z, torch.float32), dev(w, torch.float32), 64)
    torch.cuda.synchronize()
    assert err(out.cpu().numpy(), ref.out) <= TOL
    a = ssd.ssd_gated_rmsnorm_bwd(yv, dev(z, torch.float32), dev(w, torch.float32),
                                  dev(dout, torch.float32), 64)
    b = ssd.ssd_gated_rmsnorm_bwd(yv, dev(z, torch.float32), dev(w, torch.float32),
                                  dev(dout, torch.float32), 64)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_nemotron_size_sampled():
    # the Nemotron-Nano scan output's shape (8192 tokens, 64 x 64 channels, 8 norm
    # groups of 512), bf16; the oracle on a token sample (tokens are independent in
    # the forward; the weight gradient is checked in full against the oracle)
    y, z, w, dout = make(9, 1, 8192, 64, 64, True)
    out, _ = ssd.ssd_gated_rmsnorm_fwd(dev(y, torch.bfloat16), dev(z, torch.bfloat16),
                                       dev(w, torch.float32), 512, out_dtype=torch.float32)
    dy, dz, dw = ssd.ssd_gated_rmsnorm_bwd(dev(y, torch.bfloat16), dev(z, torch.bfloat16),
                                           dev(w, torch.float32), dev(dout, torch.bfloat16), 512)
    torch.cuda.synchronize()
    sel = np.arange(0, 8192, 97)
    ref = oracle.gated_rmsnorm_fwd(y[:, sel], z[:, sel], w, 512, eps=1e-5)
    assert err(out.cpu().numpy()[:, sel], ref.out) <= TOL
    g = oracle.gated_rmsnorm_bwd(y, z, w, dout, 512, eps=1e-5)
    assert err(dy.cpu().numpy(), g.dy) <= TOL
    assert err(dz.cpu().numpy(), g.dz) <= TOL
    assert err(dw.cpu().numpy(), g.dweight) <= TOL


def test_no_tokens():
    # an empty batch: nothing is written except the weight gradient, which is zero
    y = torch.empty((1, 0, 4, 16), dtype=torch.float32, device="cuda")
    w = torch.ones(64, dtype=torch.float32, device="cuda")
    out, _ = ssd.ssd_gated_rmsnorm_fwd(y, y, w, 16)
    dy, dz, dw = ssd.ssd_gated_rmsnorm_bwd(y, y, w, y, 16)
    torch.cuda.synchronize()
    assert out.shape == y.shape and dy.shape == y.shape
    assert torch.equal(dw, torch.zeros_like(dw))
