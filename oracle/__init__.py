"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the gated delta rule.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package.  It shares no code with the HIP library in
``linear_attention_gated_amd``; the two meet only at the seeded inputs.

``fwd``/``bwd`` call the plain C token-by-token recurrence in
``gdn_oracle.c`` (built with gcc, fp64, threaded over (sequence, head)).
``chunked`` holds a second, independent CPU form (the chunk-parallel WY form
in NumPy fp64) used only to check the token recurrence.

Which passage each part follows: the operator is the GatedDeltaNet core named
in the XTuner / Ascend 910C Qwen3.5-2B article, section 3.1.2 (Fig. 7 lists
the forward-state, state-gradient, dv and dq/dk/dw/dg kernels).  The article
prints no formula; the recurrence is the standard gated delta rule, stated in
``gdn_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``libgdn_oracle.so`` with gcc (plain C, fp64, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
             "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i64, dbl, p = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.gdn_oracle_fwd.argtypes = [i64, p, i64, i64, i64, dbl] + [p] * 8 + [ctypes.c_int]
        lib.gdn_oracle_fwd.restype = ctypes.c_int
        lib.gdn_oracle_bwd.argtypes = [i64, p, i64, i64, i64, dbl] + [p] * 14 + [ctypes.c_int]
        lib.gdn_oracle_bwd.restype = ctypes.c_int
        lib.gdn_oracle_threads.argtypes = [i64, i64, ctypes.c_int]
        lib.gdn_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _flat(q, k, v, g, beta, cu_seqlens):
    """Flatten [B,T,H,d] (dense) or [1,T,H,d] + cu_seqlens (varlen) to token-major
    [tokens,H,d] plus int64 cu of length N+1."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("varlen inputs must have batch 1")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    return (B * T, H, dk, dv, cu,
            _f64(q).reshape(B * T, H, dk), _f64(k).reshape(B * T, H, dk),
            _f64(v).reshape(B * T, H, dv), _f64(g).reshape(B * T, H),
            _f64(beta).reshape(B * T, H))


# In-operator L2 normalisation of q and k (optional): each (token, head) row
# x becomes x / max(||x||_2, L2_EPS).  Where ||x|| > L2_EPS the gradient is
# dx = (dy - y (y . dy)) / ||x||, the derivative of x / ||x||; below it the
# map is x / L2_EPS and dx = dy / L2_EPS.
L2_EPS = 1e-12


def l2norm_rows(x):
    """Rows of x over the last axis divided by max(||row||_2, L2_EPS), in fp64.
    Returns (y, divisor)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    d = np.maximum(n, L2_EPS)
    return x / d, d


def l2norm_rows_bwd(y, d, dy):
    """Gradient with respect to x of y = x / max(||x||, L2_EPS), given dy."""
    dy = np.asarray(dy, dtype=np.float64)
    proj = np.sum(y * dy, axis=-1, keepdims=True)
    above = d > L2_EPS
    return np.where(above, (dy - y * proj) / d, dy / L2_EPS)


def threads_used(nseq: int, heads: int, nthreads: int = 0) -> int:
    return int(_load().gdn_oracle_threads(nseq, heads, nthreads))


def fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0, nthreads=0,
        qk_l2norm=False):
    """Token-by-token forward in fp64.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; g, beta: [B,T,H]; initial_state: [N,H,dk,dv]
    holding S^T (N = B dense, or len(cu_seqlens)-1).  With ``qk_l2norm`` the
    recurrence runs on the L2-normalised rows of q and k.  Returns (o
    [B,T,H,dv], final_state [N,H,dk,dv]).
    """
    if qk_l2norm:
        q, _ = l2norm_rows(q)
        k, _ = l2norm_rows(k)
    lib = _load()
    B, T = q.shape[:2]
    NT, H, dk, dv, cu, q_, k_, v_, g_, b_ = _flat(q, k, v, g, beta, cu_seqlens)
    N = len(cu) - 1
    h0 = _f64(initial_state)
    if h0 is not None and h0.shape != (N, H, dk, dv):
        raise ValueError("initial_state shape %r != %r" % (h0.shape, (N, H, dk, dv)))
    o = np.zeros((NT, H, dv))
    ht = np.zeros((N, H, dk, dv))
    rc = lib.gdn_oracle_fwd(N, _ptr(cu), H, dk, dv, float(scale), _ptr(q_), _ptr(k_), _ptr(v_),
                            _ptr(g_), _ptr(b_), _ptr(h0), _ptr(o), _ptr(ht), int(nthreads))
    if rc != 0:
        raise MemoryError("oracle forward failed (%d)" % rc)
    return o.reshape(B, T, H, dv), ht


def bwd(q, k, v, g, beta, do, initial_state=None, dht=None, cu_seqlens=None, scale=1.0,
        nthreads=0, qk_l2norm=False):
    """Reverse-mode gradient of L = sum <do, o> + <dht, ht> through the token loop.

    With ``qk_l2norm`` the loop runs on the normalised rows and dq, dk are
    taken back through the normalisation.  Returns (dq, dk, dv, dg, dbeta,
    dh0) with the shapes of q, k, v, g, beta and the state.
    """
    if qk_l2norm:
        qh, qd = l2norm_rows(q)
        kh, kd = l2norm_rows(k)
        dqh, dkh, dv_, dg, db, dh0 = bwd(qh, kh, v, g, beta, do, initial_state, dht, cu_seqlens,
                                         scale, nthreads)
        return (l2norm_rows_bwd(qh, qd, dqh), l2norm_rows_bwd(kh, kd, dkh), dv_, dg, db, dh0)
    lib = _load()
    B, T = q.shape[:2]
    NT, H, dk, dv, cu, q_, k_, v_, g_, b_ = _flat(q, k, v, g, beta, cu_seqlens)
    N = len(cu) - 1
    h0 = _f64(initial_state)
    dht_ = _f64(dht)
    do_ = _f64(do).reshape(NT, H, dv)
    dq = np.zeros((NT, H, dk)); dk_ = np.zeros((NT, H, dk)); dv_ = np.zeros((NT, H, dv))
    dg = np.zeros((NT, H)); db = np.zeros((NT, H)); dh0 = np.zeros((N, H, dk, dv))
    rc = lib.gdn_oracle_bwd(N, _ptr(cu), H, dk, dv, float(scale), _ptr(q_), _ptr(k_), _ptr(v_),
                            _ptr(g_), _ptr(b_), _ptr(h0), _ptr(do_), _ptr(dht_), _ptr(dq),
                            _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(db), _ptr(dh0), int(nthreads))
    if rc != 0:
        raise MemoryError("oracle backward failed (%d)" % rc)
    return (dq.reshape(B, T, H, dk), dk_.reshape(B, T, H, dk), dv_.reshape(B, T, H, dv),
            dg.reshape(B, T, H), db.reshape(B, T, H), dh0)


# Gated RMSNorm on the operator's output (plain NumPy fp64; see gated_norm.py).
from .gated_norm import gated_rmsnorm_bwd, gated_rmsnorm_fwd  # noqa: E402,F401
# Causal depthwise conv1d over packed sequences (plain NumPy fp64; see conv1d.py).
from .conv1d import causal_conv1d_bwd, causal_conv1d_fwd  # noqa: E402,F401
