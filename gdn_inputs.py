"""Seeded synthetic inputs for the gated delta rule, shared by the tests, the
benchmark and the smoke check.

This module holds none of the operator's arithmetic: it only draws random
numbers, shapes them and rounds them to the working dtype.  Both the HIP path
and the CPU oracle consume what it returns; neither is imported here.

Recipe (one ``numpy.random.default_rng(seed)`` stream, PCG64, fp64 draws in the
order: sequence lengths, q, k, v, g_raw, beta_raw, h0, do):
  q, k   ~ N(0, 1), then L2-normalised over the last dim per (token, head)
  v      ~ N(0, 1)
  g      = -softplus(N(0, 1)) * g_scale          (log-decay, < 0)
  beta   = sigmoid(N(0, 1))
  h0     ~ N(0, h0_std^2) when h0_std > 0, else no initial state
  do     ~ N(0, 1) when with_grad
Each value is computed in fp64 and rounded to the storage dtype: fp32 by
round-to-nearest-even, bf16 by RNE to fp32 and then RNE to bf16.  g, beta and
states are fp32.  The arrays returned are fp64 holding exactly those rounded
values, so the oracle sees the bits the GPU sees.

Varlen lengths: L = floor(exp(U(ln lo, ln hi))) drawn until the total reaches
``total``; the last length is cut to fit (it is never zero).

Clustered keys (``k_cluster`` = sigma > 0; the stress regime of the intra-chunk
triangular solve, where beta * k_r.k_s * decay approaches 1): after the draws
above, one random unit direction u_h per head, then k = u_h + sigma * N(0, I/d)
per (token, head), L2-normalised (replacing the keys drawn above).  With
``beta_range`` = (lo, hi), beta ~ U(lo, hi) is drawn after that (replacing the
sigmoid draw).  The earlier draws are left as they are, so every other input
keeps its values.

Gated RMSNorm on the operator's output (``make_gated_norm_inputs``, its own
stream, draws in the order x, row scales, z, w, dy):
  x      ~ N(0, 1) rows times U(0.1, 3) per row, unless given (the operator's o)
  z      ~ N(0, 1.5^2)                           (the gate)
  w      = 1 + 0.1 N(0, 1), fp32                 (the norm weight, one per column)
  dy     ~ N(0, 1)                               (upstream gradient)

Causal conv1d (``make_conv_inputs``, its own stream, draws in the order
lengths, x, w, bias, dy), x channels last [B, T, C]:
  x      ~ N(0, 1)                               (the q/k/v projections)
  w      ~ U(-1/sqrt(K), 1/sqrt(K)), fp32 [C, K]  (a depthwise conv's default init range)
  bias   ~ U(-1/sqrt(K), 1/sqrt(K)), fp32 [C]
  dy     ~ N(0, 1)
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    T: int                 # per batch row (dense) or total packed tokens (varlen)
    H: int
    dk: int
    dv: int
    dtype: str             # "fp32" or "bf16"
    g_scale: float = 0.1
    h0_std: float = 0.0
    varlen: bool = False
    len_lo: int = 128
    len_hi: int = 16384
    with_grad: bool = False
    chunk: int = 64
    qk_normalized: bool = True   # False: raw q, k rows (norms spread over [0.5, 4]) for in-operator normalisation
    k_cluster: float = 0.0       # > 0: keys clustered around one direction per head (spread sigma)
    beta_range: tuple | None = None   # (lo, hi): beta ~ U(lo, hi) instead of sigmoid(N(0, 1))


# The five workloads, plus the training-step shape the throughput metric uses.
CONFIGS = {
    "c0": Config("c0_fwd_fp32_T256_H2_d64", 1, 256, 2, 64, 64, "fp32"),
    "c1": Config("c1_fwd_bf16_T4096_H16_d128", 1, 4096, 16, 128, 128, "bf16"),
    "c2": Config("c2_fwd_bf16_varlen32768_H16_d128", 1, 32768, 16, 128, 128, "bf16",
                 varlen=True),
    "c3": Config("c3_fwd_bf16_T65536_H16_d128_h0", 1, 65536, 16, 128, 128, "bf16",
                 g_scale=0.02, h0_std=0.02),
    "c4": Config("c4_fwdbwd_bf16_B2_T8192_H16_d128", 2, 8192, 16, 128, 128, "bf16",
                 with_grad=True),
    "metric": Config("fwdbwd_bf16_B1_T4096_H16_d128", 1, 4096, 16, 128, 128, "bf16",
                     with_grad=True),
}


def round_fp32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    f = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32))
    u = f.view(np.uint32)
    # RNE to the top 16 bits (in place); no overflow for finite inputs
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    u += t
    u &= np.uint32(0xFFFF0000)
    return f.astype(np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return round_fp32(x)
    raise ValueError(dtype)


def varlen_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> list:
    lens = []
    acc = 0
    while acc < total:
        L = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = max(1, min(L, total - acc))
        lens.append(L)
        acc += L
    return lens


def _l2norm(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-12)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def make_inputs(cfg: Config, seed: int = 0, *, T: int | None = None, B: int | None = None,
                H: int | None = None, lengths: list | None = None) -> dict:
    """Draw one input set.  ``T``/``B``/``H`` override the config's sizes (for
    small test cases); ``lengths`` forces the varlen sequence lengths."""
    rng = np.random.default_rng(seed)
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    cu = None
    if cfg.varlen or lengths is not None:
        if lengths is None:
            lengths = varlen_lengths(rng, T, cfg.len_lo, cfg.len_hi)
        B = 1
        T = int(sum(lengths))
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = B if cu is None else len(cu) - 1
    dt = cfg.dtype
    q = _l2norm(rng.standard_normal((B, T, H, cfg.dk)))
    k = _l2norm(rng.standard_normal((B, T, H, cfg.dk)))
    if not cfg.qk_normalized:
        q = q * rng.uniform(0.5, 4.0, (B, T, H, 1))
        k = k * rng.uniform(0.5, 4.0, (B, T, H, 1))
    v = rng.standard_normal((B, T, H, cfg.dv))
    g = -_softplus(rng.standard_normal((B, T, H))) * cfg.g_scale
    beta = _sigmoid(rng.standard_normal((B, T, H)))
    h0 = rng.standard_normal((N, H, cfg.dk, cfg.dv)) * cfg.h0_std if cfg.h0_std > 0 else None
    do = rng.standard_normal((B, T, H, cfg.dv)) if cfg.with_grad else None
    if cfg.k_cluster > 0:
        u = _l2norm(rng.standard_normal((H, cfg.dk)))
        k = _l2norm(u[None, None] + cfg.k_cluster * rng.standard_normal((B, T, H, cfg.dk)) / math.sqrt(cfg.dk))
        if not cfg.qk_normalized:
            k = k * rng.uniform(0.5, 4.0, (B, T, H, 1))
    if cfg.beta_range is not None:
        beta = rng.uniform(cfg.beta_range[0], cfg.beta_range[1], (B, T, H))
    out = dict(q=round_to(q, dt), k=round_to(k, dt), v=round_to(v, dt), g=round_fp32(g),
               beta=round_fp32(beta), h0=None if h0 is None else round_fp32(h0),
               do=None if do is None else round_to(do, dt), cu_seqlens=cu, dtype=dt,
               B=B, T=T, H=H, dk=cfg.dk, dv=cfg.dv, N=N)
    return out


def make_gated_norm_inputs(rows: int, dim: int, dtype: str, seed: int = 0, x=None) -> dict:
    """Inputs of the gated RMSNorm: x, z, dy [rows, dim] in ``dtype``, w [dim] fp32 (recipe
    in the module docstring).  ``x`` may be given (e.g. the operator's output, already
    rounded); it is then used as is."""
    rng = np.random.default_rng(seed)
    if x is None:
        x = rng.standard_normal((rows, dim)) * rng.uniform(0.1, 3.0, (rows, 1))
        x = round_to(x, dtype)
    else:
        x = np.asarray(x, dtype=np.float64).reshape(rows, dim)
    z = round_to(rng.standard_normal((rows, dim)) * 1.5, dtype)
    w = round_fp32(1.0 + 0.1 * rng.standard_normal(dim))
    dy = round_to(rng.standard_normal((rows, dim)), dtype)
    return dict(x=x, z=z, w=w, dy=dy, dtype=dtype, rows=rows, dim=dim)


def make_conv_inputs(B: int, T: int, C: int, K: int, dtype: str, seed: int = 0, *,
                     varlen_total: int | None = None, lengths=None, len_lo: int = 128,
                     len_hi: int = 16384) -> dict:
    """Inputs of the causal conv1d (recipe in the module docstring).  Packed input: give
    ``lengths`` or ``varlen_total`` (log-uniform lengths); B is then 1."""
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None or varlen_total is not None:
        if lengths is None:
            lengths = varlen_lengths(rng, varlen_total, len_lo, len_hi)
        B, T = 1, int(sum(lengths))
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x = round_to(rng.standard_normal((B, T, C)), dtype)
    bound = 1.0 / math.sqrt(K)
    w = round_fp32(rng.uniform(-bound, bound, (C, K)))
    bias = round_fp32(rng.uniform(-bound, bound, C))
    dy = round_to(rng.standard_normal((B, T, C)), dtype)
    return dict(x=x, w=w, bias=bias, dy=dy, cu_seqlens=cu, dtype=dtype, B=B, T=T, C=C, K=K)


def make_inputs_device(B: int, T: int, H: int, D: int, seed: int, device, h0_std: float = 0.02,
                       dht_std: float = 0.02, g_scale: float = 0.1) -> dict:
    """The dense bf16 workload drawn on the GPU, for shapes whose host-side fp64 draws would
    take minutes (tensors past 2^31 elements): the same distributions as make_inputs (unit
    q, k rows per head, v and do ~ N(0,1), g = -softplus(N)*g_scale, beta = sigmoid(N), h0
    and dht ~ N(0, std^2)), drawn in fp32 by torch's seeded device generator (order: q, k,
    v, g, beta, h0, do, dht) and rounded once to bf16 / fp32.  Checks read back the exact
    stored values, so the draws need not match the host generator's."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def rn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    def unit_rows(x):
        return (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)).to(torch.bfloat16)

    q = unit_rows(rn(B, T, H, D))
    k = unit_rows(rn(B, T, H, D))
    v = rn(B, T, H, D).to(torch.bfloat16)
    g = -torch.nn.functional.softplus(rn(B, T, H)) * g_scale
    beta = torch.sigmoid(rn(B, T, H))
    h0 = rn(B, H, D, D) * h0_std
    do = rn(B, T, H, D).to(torch.bfloat16)
    dht = rn(B, H, D, D) * dht_std
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, do=do, dht=dht)

