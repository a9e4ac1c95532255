"""Pins of the gated RMSNorm oracle (oracle.gated_rmsnorm_fwd / _bwd) against facts
other than itself.

* torch's own rms_norm and silu (library routines, float64 on the CPU) applied
  group by group give the same forward output.
* With weight 1 and eps 0 every group of the output has mean square exactly 1,
  and scaling y by c > 0 leaves the output unchanged.
* z = 0 closes the gate (silu(0) = 0): the output is 0.
* The gradient equals torch.autograd's gradient of the library composition, and
  central finite differences of the forward oracle along random directions.
"""
import numpy as np
import pytest
import torch

import oracle


def case(seed, b=2, T=5, H=4, P=8, gated=True):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((b, T, H, P)) * 3.0
    z = rng.standard_normal((b, T, H, P)) if gated else None
    w = rng.standard_normal(H * P)
    return y, z, w


def library_forward(y, z, w, gs, eps):
    yt = torch.as_tensor(y, dtype=torch.float64)
    g = yt if z is None else yt * torch.nn.functional.silu(torch.as_tensor(z, dtype=torch.float64))
    lead = g.shape[:-2]
    gg = g.reshape(lead + (-1, gs))
    n = torch.nn.functional.rms_norm(gg, (gs,), eps=eps)
    return (n.reshape(g.shape) * torch.as_tensor(w, dtype=torch.float64).reshape(g.shape[-2:]))


@pytest.mark.parametrize("gs", [8, 16, 32])
@pytest.mark.parametrize("gated", [True, False])
def test_forward_matches_library_composition(gs, gated):
    y, z, w = case(1, gated=gated)
    r = oracle.gated_rmsnorm_fwd(y, z, w, gs, eps=1e-5)
    ref = library_forward(y, z, w, gs, 1e-5).numpy()
    assert np.max(np.abs(r.out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_unit_mean_square_and_scale_invariance():
    y, z, _ = case(2)
    ones = np.ones(4 * 8)
    r = oracle.gated_rmsnorm_fwd(y, z, ones, 16, eps=0.0)
    ms = np.mean(r.out.reshape(2, 5, 2, 16) ** 2, axis=-1)
    assert np.max(np.abs(ms - 1.0)) <= 1e-13
    r2 = oracle.gated_rmsnorm_fwd(7.5 * y, z, ones, 16, eps=0.0)
    assert np.max(np.abs(r2.out - r.out)) <= 1e-13


def test_closed_gate_gives_zero():
    y, _, w = case(3)
    r = oracle.gated_rmsnorm_fwd(y, np.zeros_like(y), w, 16, eps=1e-5)
    assert np.all(r.out == 0.0)


@pytest.mark.parametrize("gated", [True, False])
def test_backward_matches_autograd_of_library(gated):
    y, z, w = case(4, gated=gated)
    dout = np.random.default_rng(5).standard_normal(y.shape)
    gs, eps = 16, 1e-5
    g = oracle.gated_rmsnorm_bwd(y, z, w, dout, gs, eps=eps)
    yt = torch.tensor(y, requires_grad=True)
    zt = torch.tensor(z, requires_grad=True) if gated else None
    wt = torch.tensor(w, requires_grad=True)
    gt = yt if zt is None else yt * torch.nn.functional.silu(zt)
    n = torch.nn.functional.rms_norm(gt.reshape(2, 5, -1, gs), (gs,), eps=eps)
    out = n.reshape(gt.shape) * wt.reshape(4, 8)
    (out * torch.tensor(dout)).sum().backward()
    assert np.max(np.abs(g.dy - yt.grad.numpy())) <= 1e-12 * np.max(np.abs(g.dy))
    assert np.max(np.abs(g.dweight - wt.grad.numpy())) <= 1e-12 * np.max(np.abs(g.dweight))
    if gated:
        assert np.max(np.abs(g.dz - zt.grad.numpy())) <= 1e-12 * np.max(np.abs(g.dz))


def test_backward_finite_differences():
    y, z, w = case(6)
    rng = np.random.default_rng(7)
    dout = rng.standard_normal(y.shape)
    gs, eps, h = 8, 1e-5, 1e-6
    g = oracle.gated_rmsnorm_bwd(y, z, w, dout, gs, eps=eps)
    L = lambda yy, zz, ww: float(np.sum(dout * oracle.gated_rmsnorm_fwd(yy, zz, ww, gs, eps).out))
    for name, grad in (("y", g.dy), ("z", g.dz), ("w", g.dweight)):
        d = rng.standard_normal(grad.shape)
        args = {"y": y, "z": z, "w": w}
        plus, minus = dict(args), dict(args)
        plus[name] = args[name] + h * d
        minus[name] = args[name] - h * d
        fd = (L(plus["y"], plus["z"], plus["w"]) - L(minus["y"], minus["z"], minus["w"])) / (2 * h)
        an = float(np.sum(grad * d))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


# ------------------------------------------------------------------ planted slips
#
# Each mutant is the oracle's forward or gradient with one plausible slip; the
# library composition (torch rms_norm / silu / autograd) must reject every one.

def _mut_fwd(kind, y, z, w, gs, eps):
    y = np.asarray(y, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-z))
    g = {"sigmoid_gate": y * s, "norm_before_gate": y}.get(kind, y * z * s)
    lead = y.shape[:-2]
    gg = g.reshape(lead + (-1, gs))
    if kind == "group_over_heads_axis":
        gg = g.reshape(lead + (gs, -1)).swapaxes(-1, -2)
    ms = np.mean(gg * gg, axis=-1)
    if kind == "no_eps":
        eps = 0.0
    r = 1.0 / np.sqrt(ms + eps) if kind != "std_not_rms" else 1.0 / np.sqrt(
        np.var(gg, axis=-1) + eps)
    xh = gg * r[..., None]
    if kind == "group_over_heads_axis":
        xh = xh.swapaxes(-1, -2)
    out = xh.reshape(y.shape)
    if kind == "norm_before_gate":
        out = out * z * s
    return out * np.asarray(w).reshape(y.shape[-2:])


@pytest.mark.parametrize("kind", ["sigmoid_gate", "norm_before_gate", "no_eps",
                                  "std_not_rms", "group_over_heads_axis"])
def test_forward_slips_are_caught(kind):
    y, z, w = case(8)
    y = y * 1e-3  # small activations make a dropped eps visible
    ref = library_forward(y, z, w, 16, 1e-5).numpy()
    bad = _mut_fwd(kind, y, z, w, 16, 1e-5)
    assert np.max(np.abs(bad - ref)) > 1e-6 * np.max(np.abs(ref))


def _mut_bwd(kind, y, z, w, dout, gs, eps):
    g = oracle.gated_rmsnorm_bwd(y, z, w, dout, gs, eps)
    sig = 1.0 / (1.0 + np.exp(-z))
    if kind == "dz_without_product_rule":
        dg = g.dy / (z * sig)
        return g.dy, dg * y * sig, g.dweight
    if kind == "dy_without_gate":
        return g.dy / (z * sig), g.dz, g.dweight
    if kind == "dweight_on_gated_not_normalised":
        gg = (y * z * sig)
        return g.dy, g.dz, np.sum((dout * gg).reshape(-1, w.size), axis=0)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["dz_without_product_rule", "dy_without_gate",
                                  "dweight_on_gated_not_normalised"])
def test_gradient_slips_are_caught(kind):
    y, z, w = case(9)
    dout = np.random.default_rng(10).standard_normal(y.shape)
    dy, dz, dw = _mut_bwd(kind, y, z, w, dout, 16, 1e-5)
    yt = torch.tensor(y, requires_grad=True)
    zt = torch.tensor(z, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    n = torch.nn.functional.rms_norm((yt * torch.nn.functional.silu(zt)).reshape(2, 5, -1, 16),
                                     (16,), eps=1e-5)
    (n.reshape(yt.shape) * wt.reshape(4, 8) * torch.tensor(dout)).sum().backward()
    bad = max(np.max(np.abs(dy - yt.grad.numpy())), np.max(np.abs(dz - zt.grad.numpy())),
              np.max(np.abs(dw - wt.grad.numpy())))
    assert bad > 1e-6
