"""The oracle against exact rational arithmetic on tiny inputs, and against its
stored regression fixture.  CPU only.

With g = 0 (so the decay factor is exactly 1) and dyadic inputs, every
quantity of the delta rule is an exact rational; the fp64 oracle must agree to
rounding.  The exact evaluation below uses the matrix-product form
S_t = S_{t-1} (I - beta k k^T) + beta v k^T with Python Fractions, a different
computation from the oracle's element loops.
"""
import json
import os
from fractions import Fraction as Fr

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _matmul(A, B):
    return [[sum(A[i][x] * B[x][j] for x in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def test_exact_rational_forward():
    rng = np.random.default_rng(7)
    T, dk, dv = 6, 3, 2
    # dyadic values: integers / 8
    q = rng.integers(-8, 9, (T, dk)) / 8.0
    k = rng.integers(-8, 9, (T, dk)) / 8.0
    v = rng.integers(-8, 9, (T, dv)) / 8.0
    beta = rng.integers(0, 5, T) / 4.0
    S0 = rng.integers(-8, 9, (dv, dk)) / 8.0
    S = [[Fr(x) for x in row] for row in S0]
    outs = []
    for t in range(T):
        kt = [Fr(x) for x in k[t]]
        M = [[(Fr(1) if i == j else Fr(0)) - Fr(beta[t]) * kt[i] * kt[j] for j in range(dk)]
             for i in range(dk)]
        S = _matmul(S, M)
        S = [[S[j][i] + Fr(beta[t]) * Fr(v[t][j]) * kt[i] for i in range(dk)] for j in range(dv)]
        outs.append([sum(S[j][i] * Fr(q[t][i]) for i in range(dk)) for j in range(dv)])
    o, ht = oracle.fwd(q[None, :, None], k[None, :, None], v[None, :, None],
                       np.zeros((1, T, 1)), beta[None, :, None], S0.T[None, None])
    exact_o = np.array([[float(x) for x in row] for row in outs])
    exact_ht = np.array([[float(S[j][i]) for j in range(dv)] for i in range(dk)])
    assert np.max(np.abs(o[0, :, 0] - exact_o)) < 1e-13
    assert np.max(np.abs(ht[0, 0] - exact_ht)) < 1e-13


def test_regression_fixture():
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        c = json.load(f)
    a = {key: np.array(val) for key, val in c.items() if key not in ("expected", "scale")}
    o, ht = oracle.fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], scale=c["scale"])
    grads = oracle.bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["do"], a["h0"], a["dht"],
                       scale=c["scale"])
    exp = c["expected"]
    assert np.allclose(o, exp["o"], rtol=0, atol=1e-12)
    assert np.allclose(ht, exp["ht"], rtol=0, atol=1e-12)
    for name, val in zip("dq dk dv dg dbeta dh0".split(), grads):
        assert np.allclose(val, exp[name], rtol=0, atol=1e-12), name
