"""Pins of the fp64 causal-conv1d oracle (oracle/conv1d.py): PyTorch's own fp64
conv1d (padding K-1, groups = channels, the first T outputs) with silu and its
autograd, per sequence; no leakage across sequence starts; the impulse
response; K = 1; varlen equals separate dense calls; finite differences."""
import numpy as np
import pytest
import torch

import oracle

R = np.random.default_rng(11)


def torch_ref(x, w, bias, act, lens, dy):
    """Per sequence: conv1d with K-1 zeros of left padding, then silu; gradients by autograd."""
    ys, dxs = [], []
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    bt = None if bias is None else torch.tensor(bias, dtype=torch.float64, requires_grad=True)
    C, K = w.shape
    a = 0
    for n in lens:
        if n == 0:   # an empty sequence contributes nothing
            continue
        xs = torch.tensor(x[a:a + n], dtype=torch.float64, requires_grad=True)
        pre = torch.nn.functional.conv1d(xs.T[None], wt[:, None, :], bt, padding=K - 1, groups=C)[0, :, :n].T
        y = torch.nn.functional.silu(pre) if act else pre
        y.backward(torch.tensor(dy[a:a + n]))
        ys.append(y.detach().numpy())
        dxs.append(xs.grad.numpy())
        a += n
    return (np.concatenate(ys) if ys else np.zeros((0, C)), np.concatenate(dxs) if dxs else np.zeros((0, C)),
            wt.grad.numpy() if wt.grad is not None else np.zeros_like(w),
            None if bt is None else (bt.grad.numpy() if bt.grad is not None else np.zeros(C)))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("act,with_bias", [(True, True), (False, False), (True, False)])
def test_matches_torch_conv1d_per_sequence(K, act, with_bias):
    lens = [5, 1, 0, 2, 9, 3]
    T, C = sum(lens), 6
    x = R.standard_normal((T, C))
    w = R.standard_normal((C, K))
    b = R.standard_normal(C) if with_bias else None
    dy = R.standard_normal((T, C))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    y = oracle.causal_conv1d_fwd(x[None], w, b, cu, act)[0]
    dx, dw, db = oracle.causal_conv1d_bwd(x[None], w, dy[None], b, cu, act)
    ry, rdx, rdw, rdb = torch_ref(x, w, b, act, lens, dy)
    np.testing.assert_allclose(y, ry, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dx[0], rdx, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, rdw, rtol=1e-12, atol=1e-12)
    if with_bias:
        np.testing.assert_allclose(db, rdb, rtol=1e-12, atol=1e-12)
    else:
        # the bias gradient is defined also without a bias: the sum of dpre
        _, _, _, rdb0 = torch_ref(x, w, np.zeros(C), act, lens, dy)
        np.testing.assert_allclose(db, rdb0, rtol=1e-12, atol=1e-12)


def test_no_leakage_across_sequence_starts():
    lens = [7, 4, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = R.standard_normal((1, 17, 3))
    w, b, dy = R.standard_normal((3, 4)), R.standard_normal(3), R.standard_normal((1, 17, 3))
    y = oracle.causal_conv1d_fwd(x, w, b, cu)
    dx = oracle.causal_conv1d_bwd(x, w, dy, b, cu)[0]
    x2 = x.copy()
    x2[0, 7:11] += 5.0          # the middle sequence only
    dy2 = dy.copy()
    dy2[0, 7:11] -= 3.0
    y2 = oracle.causal_conv1d_fwd(x2, w, b, cu)
    dx2 = oracle.causal_conv1d_bwd(x2, w, dy2, b, cu)[0]
    for sl in (slice(0, 7), slice(11, 17)):
        assert np.array_equal(y[0, sl], y2[0, sl])
        assert np.array_equal(dx[0, sl], dx2[0, sl])


def test_impulse_response_and_k1():
    C, K, T = 2, 4, 10
    w = R.standard_normal((C, K))
    x = np.zeros((1, T, C))
    x[0, 3, 1] = 1.0
    y = oracle.causal_conv1d_fwd(x, w, None, None, activation=False)[0]
    # an impulse at t = 3 gives w[c, K-1-s] at t = 3 + s, nothing else
    want = np.zeros((T, C))
    for s in range(K):
        want[3 + s, 1] = w[1, K - 1 - s]
    assert np.array_equal(y, want)
    w1 = R.standard_normal((C, 1))
    b1 = R.standard_normal(C)
    xr = R.standard_normal((2, T, C))
    y1 = oracle.causal_conv1d_fwd(xr, w1, b1)
    pre = xr * w1[:, 0] + b1
    np.testing.assert_allclose(y1, pre / (1 + np.exp(-pre)), rtol=1e-14)


def test_varlen_equals_separate_dense_calls():
    lens = [3, 8, 1, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = R.standard_normal((1, sum(lens), 4))
    dy = R.standard_normal(x.shape)
    w, b = R.standard_normal((4, 3)), R.standard_normal(4)
    y = oracle.causal_conv1d_fwd(x, w, b, cu)
    dx, dw, db = oracle.causal_conv1d_bwd(x, w, dy, b, cu)
    dws, dbs = np.zeros_like(dw), np.zeros_like(db)
    for i, n in enumerate(lens):
        sl = slice(cu[i], cu[i + 1])
        yi = oracle.causal_conv1d_fwd(x[:, sl], w, b)
        dxi, dwi, dbi = oracle.causal_conv1d_bwd(x[:, sl], w, dy[:, sl], b)
        assert np.array_equal(y[:, sl], yi) and np.array_equal(dx[:, sl], dxi)
        dws += dwi
        dbs += dbi
    np.testing.assert_allclose(dw, dws, rtol=1e-13)
    np.testing.assert_allclose(db, dbs, rtol=1e-13)


def test_finite_differences():
    lens = [4, 6]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = R.standard_normal((1, 10, 3))
    w, b, dy = R.standard_normal((3, 4)), R.standard_normal(3), R.standard_normal((1, 10, 3))
    dx, dw, db = oracle.causal_conv1d_bwd(x, w, dy, b, cu)
    h = 1e-6

    def loss(x_, w_, b_):
        return np.sum(dy * oracle.causal_conv1d_fwd(x_, w_, b_, cu))

    for name, g, base in (("x", dx, x), ("w", dw, w), ("b", db, b)):
        for _ in range(3):
            d = R.standard_normal(base.shape)
            args_p, args_m = [x, w, b], [x, w, b]
            i = ("x", "w", "b").index(name)
            args_p[i] = base + h * d
            args_m[i] = base - h * d
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            an = np.sum(g * d)
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)
