"""TEST INFRASTRUCTURE ONLY: fp64 CPU oracle of the gated RMSNorm on the
operator's output.  Only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s CPU-baseline leg may import it; it shares no code with the HIP
library.

Passages followed: the XTuner / Ascend 910C Qwen3.5 training article, §2.4
(the 1 ms window of Fig. 3C, decoded there as the output gate's RMSNorm taken
apart term by term: the row cast to fp32, its squares, their mean, plus eps,
the reciprocal square root, the product with the row, the product with the
weight, then the gate's SiLU and the product with it) and §3.1.2 (Fig. 6 and
Fig. 9: the same chain as one fused forward kernel and one backward kernel).

Per (token, head) row x of length d, with gate row z of the same length and a
weight w of length d shared by all rows:

    r = (mean_i x_i^2 + eps)^(-1/2),   n = r x,   a = n * w,
    y = a * silu(z),                  silu(z) = z * sigmoid(z).

Backward, for an upstream gradient dy (the derivative of each line above):

    da = dy * silu(z)              dz = dy * a * sigmoid(z) * (1 + z (1 - sigmoid(z)))
    dw = sum over rows of da * n   dn = da * w
    dx = r (dn - n * mean_i(dn_i n_i))

Everything is fp64 here; the pages fix no precision beyond computing the
variance in fp32.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def _sigmoid(z):
    # both branches from exp(-|z|), so neither overflows
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gated_rmsnorm_fwd(x, z, w, eps=EPS):
    """y = (x * (mean(x^2) + eps)^(-1/2) * w) * silu(z) over the last axis, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = x * r
    return n * w * (z * _sigmoid(z))


def gated_rmsnorm_bwd(x, z, w, dy, eps=EPS):
    """Gradients (dx, dz, dw) of sum(dy * y) for y = gated_rmsnorm_fwd(x, z, w, eps).
    dw sums over every row (all leading axes)."""
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    d = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = x * r
    a = n * w
    s = _sigmoid(z)
    da = dy * (z * s)
    dz = dy * a * s * (1.0 + z * (1.0 - s))
    dw = np.sum((da * n).reshape(-1, d), axis=0)
    dn = da * w
    dx = r * (dn - n * np.mean(dn * n, axis=-1, keepdims=True))
    return dx, dz, dw
