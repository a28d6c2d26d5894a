"""Pins of the fp64 gated-RMSNorm oracle (oracle/gated_norm.py) against what the
mathematics fixes: PyTorch's own fp64 CPU rms_norm/silu and autograd (an
independent library implementation), scale invariance, unit RMS, the gradient's
orthogonality to the row, the zero gate, zero rows and finite differences."""
import numpy as np
import pytest
import torch

import oracle

R = np.random.default_rng(7)


def inputs(shape=(3, 5, 2, 16), eps=1e-6, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * rng.uniform(0.1, 3.0, shape[:-1] + (1,))
    z = rng.standard_normal(shape) * 2.0
    w = 1.0 + 0.3 * rng.standard_normal(shape[-1])
    dy = rng.standard_normal(shape)
    return x, z, w, dy, eps


@pytest.mark.parametrize("eps", [1e-6, 1e-2, 0.0])
def test_matches_torch_rms_norm_silu_and_autograd(eps):
    x, z, w, dy, _ = inputs()
    xt, zt, wt = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, z, w))
    yt = torch.nn.functional.rms_norm(xt, (x.shape[-1],), wt, eps=eps) * torch.nn.functional.silu(zt)
    yt.backward(torch.tensor(dy))
    y = oracle.gated_rmsnorm_fwd(x, z, w, eps)
    dx, dz, dw = oracle.gated_rmsnorm_bwd(x, z, w, dy, eps)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_scale_invariance_and_unit_rms_without_eps():
    x, z, w, dy, _ = inputs()
    c = np.exp(R.uniform(-3, 3, x.shape[:-1] + (1,)))
    np.testing.assert_allclose(oracle.gated_rmsnorm_fwd(c * x, z, w, 0.0),
                               oracle.gated_rmsnorm_fwd(x, z, w, 0.0), rtol=1e-12, atol=1e-14)
    # w = 1 and a gate where silu(z) = z sigmoid(z) is known: y / silu(z) has unit RMS
    zc = np.full_like(x, 3.0)
    y = oracle.gated_rmsnorm_fwd(x, zc, np.ones(x.shape[-1]), 0.0)
    n = y / (3.0 / (1.0 + np.exp(-3.0)))
    np.testing.assert_allclose(np.mean(n * n, axis=-1), 1.0, rtol=1e-12)


def test_gradient_orthogonal_to_row_without_eps():
    x, z, w, dy, _ = inputs()
    dx, _, _ = oracle.gated_rmsnorm_bwd(x, z, w, dy, 0.0)
    dots = np.sum(dx * x, axis=-1)
    scale = np.linalg.norm(dx, axis=-1) * np.linalg.norm(x, axis=-1)
    assert np.max(np.abs(dots) / scale) < 1e-12


def test_zero_gate_and_zero_rows():
    x, z, w, dy, eps = inputs()
    z0 = np.zeros_like(z)
    assert np.all(oracle.gated_rmsnorm_fwd(x, z0, w, eps) == 0)
    dx, dz, dw = oracle.gated_rmsnorm_bwd(x, z0, w, dy, eps)
    assert np.all(dx == 0) and np.all(dw == 0)
    # silu'(0) = 1/2: dz = dy * a / 2 with a the weighted normalised row
    a = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w
    np.testing.assert_allclose(dz, 0.5 * dy * a, rtol=1e-13)
    # a zero row: y = 0 and dx = dn / sqrt(eps) (the mean term vanishes with n = 0)
    xz = x.copy()
    xz[1, 2, 0] = 0.0
    assert np.all(oracle.gated_rmsnorm_fwd(xz, z, w, eps)[1, 2, 0] == 0)
    dx, _, _ = oracle.gated_rmsnorm_bwd(xz, z, w, dy, eps)
    s = 1.0 / (1.0 + np.exp(-z[1, 2, 0]))
    np.testing.assert_allclose(dx[1, 2, 0], dy[1, 2, 0] * z[1, 2, 0] * s * w / np.sqrt(eps), rtol=1e-12)


def test_finite_differences():
    x, z, w, dy, eps = inputs(shape=(2, 3, 8), eps=1e-3, seed=3)
    dx, dz, dw = oracle.gated_rmsnorm_bwd(x, z, w, dy, eps)
    h = 1e-6

    def loss(x_, z_, w_):
        return np.sum(dy * oracle.gated_rmsnorm_fwd(x_, z_, w_, eps))

    for which, g in (("x", dx), ("z", dz), ("w", dw)):
        for _ in range(3):
            dirn = R.standard_normal(g.shape)
            args_p = {"x": x, "z": z, "w": w}
            args_m = dict(args_p)
            args_p[which] = args_p[which] + h * dirn
            args_m[which] = args_m[which] - h * dirn
            fd = (loss(**{k + "_": v for k, v in args_p.items()}) -
                  loss(**{k + "_": v for k, v in args_m.items()})) / (2 * h)
            an = np.sum(g * dirn)
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_sigmoid_saturation_is_finite():
    x, z, w, dy, eps = inputs()
    zs = np.where(R.random(z.shape) < 0.5, 800.0, -800.0)
    y = oracle.gated_rmsnorm_fwd(x, zs, w, eps)
    dx, dz, dw = oracle.gated_rmsnorm_bwd(x, zs, w, dy, eps)
    assert all(np.all(np.isfinite(a)) for a in (y, dx, dz, dw))
    # silu(-800) = 0 to double precision, silu(800) = 800
    a = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w
    np.testing.assert_allclose(y, np.where(zs > 0, 800.0 * a, 0.0), rtol=1e-14, atol=0)
