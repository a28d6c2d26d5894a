"""TEST INFRASTRUCTURE ONLY: fp64 CPU oracle of the causal depthwise conv1d
(with optional SiLU) over packed variable-length sequences.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it;
it shares no code with the HIP library.

Passages followed: the XTuner / Ascend 910C Qwen3.5 training article, §3.1.2
(the GDN stack's causal conv1d, first run as a loop of slices and pads per
sequence, then as one native forward and one backward kernel, Fig. 8).  The
article prints no formula; this is the short causal convolution of the GDN
layer: per channel c, kernel size K, for token t of a sequence that starts at
token t0,

    pre[t, c] = bias[c] + sum_{j=0}^{K-1} w[c, j] * x[t - (K-1) + j, c],
                with x[t', c] = 0 for t' < t0 (nothing crosses a sequence start),
    y[t, c]   = silu(pre[t, c])  (or pre[t, c] without the activation).

Backward for dy:  dpre = dy * silu'(pre) (or dy),
    dx[t', c]   = sum_j w[c, j] * dpre[t' + (K-1) - j, c]   (same sequence only),
    dw[c, j]    = sum_t dpre[t, c] * x[t - (K-1) + j, c],    dbias[c] = sum_t dpre[t, c].
Everything is fp64.
"""
from __future__ import annotations

import numpy as np


def _sigmoid(u):
    e = np.exp(-np.abs(u))
    return np.where(u >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def _sequences(x, cu_seqlens):
    """(start, end) token ranges of the sequences of x [B, T, C] (dense) or [1, T, C] + cu."""
    B, T, _ = x.shape
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    if B != 1:
        raise ValueError("varlen inputs must have batch 1")
    cu = [int(c) for c in cu_seqlens]
    return list(zip(cu[:-1], cu[1:]))


def _shifted(xs, s):
    """xs delayed by s tokens within one sequence: row t holds xs[t - s], zeros before the start."""
    out = np.zeros_like(xs)
    if s < xs.shape[0]:
        out[s:] = xs[:xs.shape[0] - s]
    return out


def causal_conv1d_fwd(x, w, bias=None, cu_seqlens=None, activation=True):
    """y [B, T, C] (fp64) for x [B, T, C], w [C, K], bias [C] or None."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, C = x.shape
    K = w.shape[1]
    flat = x.reshape(B * T, C)
    y = np.zeros_like(flat)
    for a, b in _sequences(x, cu_seqlens):
        xs = flat[a:b]
        pre = np.zeros_like(xs) + (0.0 if bias is None else np.asarray(bias, dtype=np.float64))
        for j in range(K):
            pre += w[:, j] * _shifted(xs, K - 1 - j)
        y[a:b] = pre * _sigmoid(pre) if activation else pre
    return y.reshape(B, T, C)


def causal_conv1d_bwd(x, w, dy, bias=None, cu_seqlens=None, activation=True):
    """(dx [B, T, C], dw [C, K], dbias [C]) for L = sum(dy * y)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    B, T, C = x.shape
    K = w.shape[1]
    flat, gflat = x.reshape(B * T, C), dy.reshape(B * T, C)
    dx = np.zeros_like(flat)
    dw = np.zeros((C, K))
    db = np.zeros(C)
    for a, b in _sequences(x, cu_seqlens):
        xs, gs = flat[a:b], gflat[a:b]
        n = b - a
        pre = np.zeros_like(xs) + (0.0 if bias is None else np.asarray(bias, dtype=np.float64))
        for j in range(K):
            pre += w[:, j] * _shifted(xs, K - 1 - j)
        if activation:
            s = _sigmoid(pre)
            dpre = gs * s * (1.0 + pre * (1.0 - s))
        else:
            dpre = gs
        db += dpre.sum(axis=0)
        for j in range(K):
            d = K - 1 - j
            dw[:, j] += np.sum(dpre * _shifted(xs, d), axis=0)
            # dx[t'] gets w[:, j] * dpre[t' + d] when t' + d is still in the sequence
            if d < n:
                dx[a:b - d] += w[:, j] * dpre[d:]
    return dx.reshape(B, T, C), dw, db
