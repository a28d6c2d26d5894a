"""GPU parity of the backward pass (HIP path through the C ABI) against the
fp64 oracle's reverse-mode token loop, element by element, on seeded inputs."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
import oracle
from gpu_util import (TOL, batch_in_one_round, batch_past_one_round, device_cus, dev_inputs, frob, maxrel, say,
                      small_cfg, to_np)

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def run_bwd(x, dht=None, scale=1.0, use_context=True, l2=False):
    d = dev_inputs(x)
    dht_t = None if dht is None else torch.from_numpy(dht).float().cuda()
    ctx = None
    if use_context:
        _, _, ctx = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"],
                            cu_seqlens=d["cu"], scale=scale, return_context=True, qk_l2norm=l2)
    r = gdn.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], initial_state=d["h0"],
                dht=dht_t, cu_seqlens=d["cu"], scale=scale, context=ctx, qk_l2norm=l2)
    torch.cuda.synchronize()
    return [to_np(t) for t in r]


def ref_bwd(x, dht=None, scale=1.0, l2=False):
    return oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], x["h0"], dht,
                      cu_seqlens=x["cu_seqlens"], scale=scale, qk_l2norm=l2)


def compare(x, dht=None, scale=1.0, label="", use_context=True, l2=False):
    say("case", label, "dtype", x["dtype"], "B", x["B"], "T", x["T"], "H", x["H"], "d", x["dk"],
        "N", x["N"], "context", use_context, "qk_l2norm", l2)
    got = run_bwd(x, dht, scale, use_context, l2)
    ref = ref_bwd(x, dht, scale, l2)
    tol = TOL[x["dtype"]]
    bad = []
    for name, a, b in zip(NAMES, got, ref):
        mr, fr = maxrel(a, b), frob(a, b)
        say("  %-6s maxrel %.3e  frob %.3e" % (name, mr, fr))
        if not np.all(np.isfinite(a)):
            bad.append(name + " non-finite")
        elif mr > tol["maxrel"] or fr > tol["frob"]:
            bad.append("%s maxrel %.2e frob %.2e" % (name, mr, fr))
    assert not bad, bad
    return got


def test_config0_shape_fp32_backward():
    cfg = gi.Config("c0_bwd", 1, 256, 2, 64, 64, "fp32", with_grad=True)
    compare(gi.make_inputs(cfg, 0), label="c0 shape fwd+bwd fp32")


SMALL = [
    ("fp32", 64, 1, 200, 3, 0.0, False, 0.7),
    ("fp32", 64, 2, 130, 2, 0.3, True, 1.0),
    ("fp32", 64, 1, 1, 2, 0.5, True, 1.0),
    ("fp32", 128, 1, 200, 2, 0.2, True, 0.8),
    ("fp32", 128, 2, 65, 1, 0.0, False, 1.0),
    ("fp32", 128, 1, 1, 1, 0.3, True, 1.0),
    ("bf16", 64, 2, 300, 2, 0.0, False, 1.0),
    ("bf16", 128, 1, 257, 3, 0.2, True, 1.0),
    ("bf16", 128, 1, 63, 1, 0.0, False, 0.125),
    ("bf16", 128, 1, 64, 2, 0.0, True, 1.0),
    ("bf16", 128, 2, 65, 2, 0.1, False, 1.0),
]


@pytest.mark.parametrize("dtype,d,B,T,H,h0,with_dht,scale", SMALL)
def test_small_dense(dtype, d, B, T, H, h0, with_dht, scale):
    cfg = small_cfg(dtype, d, B=B, T=T, H=H, h0_std=h0, with_grad=True)
    x = gi.make_inputs(cfg, 11)
    dht = np.random.default_rng(3).standard_normal((x["N"], H, d, d)) * 0.1 if with_dht else None
    compare(x, dht=dht, scale=scale, label="small")


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128), ("fp32", 128)])
def test_decay_extremes(dtype, d):
    # per-token log decays of exactly 0 (no forgetting), -30 (exp(g) ~ 1e-13: the chunk's
    # cumulative decays underflow to 0 within a few tokens) and the usual draws, in runs
    # that straddle chunk boundaries; the backward must stay finite and match the oracle
    cfg = small_cfg(dtype, d, T=300, H=2, h0_std=0.2, with_grad=True)
    x = gi.make_inputs(cfg, 13)
    rng = np.random.default_rng(14)
    runs = np.repeat(rng.integers(0, 3, size=(x["B"], 300 // 25 + 1, x["H"])), 25, axis=1)[:, :300]
    x["g"] = np.where(runs == 0, 0.0, np.where(runs == 1, -30.0, x["g"]))
    dht = np.random.default_rng(15).standard_normal((x["N"], 2, d, d)) * 0.1
    compare(x, dht=dht, label="decay 0 / -30 / drawn")


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128), ("fp32", 128)])
def test_small_varlen(dtype, d):
    cfg = small_cfg(dtype, d, H=2, h0_std=0.3, with_grad=True)
    x = gi.make_inputs(cfg, 12, lengths=[1, 0, 63, 64, 65, 130, 0, 7])
    dht = np.random.default_rng(4).standard_normal((x["N"], 2, d, d)) * 0.1
    got = compare(x, dht=dht, label="varlen")
    # empty sequences pass the state gradient through
    assert np.array_equal(got[5][1], dht[1].astype(np.float32))
    assert np.array_equal(got[5][6], dht[6].astype(np.float32))


def test_recompute_equals_saved_context():
    cfg = small_cfg("bf16", 128, T=200, H=2, h0_std=0.1, with_grad=True)
    x = gi.make_inputs(cfg, 13)
    a = run_bwd(x, use_context=True)
    b = run_bwd(x, use_context=False)
    for n, u, v in zip(NAMES, a, b):
        assert np.array_equal(u, v), n


def test_bitwise_deterministic_backward():
    cfg = small_cfg("bf16", 128, T=190, H=3, with_grad=True)
    x = gi.make_inputs(cfg, 14)
    a = run_bwd(x)
    b = run_bwd(x)
    for n, u, v in zip(NAMES, a, b):
        assert np.array_equal(u, v), n


def test_fp32_head_dim_128_config0_shape_and_recompute():
    # fp32 at d = 128: the gradient kernel reads Q and K from global memory and stores its
    # outputs directly (the staged tiles would not fit the LDS); T = 256, H = 2 as the fp32
    # workload, with h0 and dht; recomputing the forward context gives the same bits
    cfg = gi.Config("fp32_d128_bwd", 1, 256, 2, 128, 128, "fp32", h0_std=0.1, with_grad=True)
    x = gi.make_inputs(cfg, 15)
    dht = np.random.default_rng(16).standard_normal((1, 2, 128, 128)) * 0.1
    a = compare(x, dht=dht, label="fp32 d=128 fwd+bwd")
    b = run_bwd(x, dht=dht, use_context=False)
    for n, u, v in zip(NAMES, a, b):
        assert np.array_equal(u, v), n


@pytest.mark.parametrize("name", ["metric", "c4"])
def test_full_fwd_bwd(name):
    x = gi.make_inputs(gi.CONFIGS[name], 0)
    compare(x, label=name)


def test_full_packed_varlen_fwd_bwd():
    # the packed workload (32768 tokens in log-uniform sequences, H=16, d=128) with do
    import dataclasses
    cfg = dataclasses.replace(gi.CONFIGS["c2"], name="c2_fwdbwd", with_grad=True)
    x = gi.make_inputs(cfg, 0)
    assert x["N"] > 1 and x["cu_seqlens"] is not None
    compare(x, label="c2 packed fwd+bwd")


def test_thousands_of_short_sequences():
    # 2500 sequences of 0..80 tokens: the planner's scan runs three passes of 1024 sequences
    # (with the carry between them), empty sequences pass h0 through, most chunks are partial
    lengths = [int(v) for v in np.random.default_rng(23).integers(0, 81, 2500)]
    lengths[:5] = [0, 0, 1, 64, 65]
    cfg = small_cfg("bf16", 64, H=2, h0_std=0.05, with_grad=True)
    x = gi.make_inputs(cfg, 24, lengths=lengths)
    assert x["N"] == 2500
    dht = np.random.default_rng(25).standard_normal((x["N"], 2, 64, 64)) * 0.05
    compare(x, dht=dht, scale=0.5, label="2500 packed sequences")


def test_packed_varlen_with_states_and_scale():
    # packed sequences with initial states, a final-state gradient and scale != 1
    cfg = small_cfg("bf16", 128, H=3, h0_std=0.05, with_grad=True)
    x = gi.make_inputs(cfg, 21, lengths=[300, 1, 64, 0, 777, 129, 5])
    dht = np.random.default_rng(22).standard_normal((x["N"], 3, 128, 128)) * 0.05
    compare(x, dht=dht, scale=0.3, label="packed h0 dht scale")



# in-operator L2 normalisation of q and k, on raw rows
L2 = [
    ("fp32", 64, 1, 150, 2, 0.2, True, 0.9),
    ("fp32", 128, 1, 130, 2, 0.1, True, 1.0),
    ("bf16", 64, 2, 130, 2, 0.0, False, 1.0),
    ("bf16", 128, 1, 200, 3, 0.1, True, 1.0),
]


@pytest.mark.parametrize("dtype,d,B,T,H,h0,with_dht,scale", L2)
def test_l2norm_small(dtype, d, B, T, H, h0, with_dht, scale):
    cfg = small_cfg(dtype, d, B=B, T=T, H=H, h0_std=h0, with_grad=True, qk_normalized=False)
    x = gi.make_inputs(cfg, 41)
    dht = np.random.default_rng(5).standard_normal((x["N"], H, d, d)) * 0.1 if with_dht else None
    compare(x, dht=dht, scale=scale, label="l2norm", l2=True)


def test_l2norm_varlen_and_recompute():
    cfg = small_cfg("bf16", 128, H=2, h0_std=0.1, with_grad=True, qk_normalized=False)
    x = gi.make_inputs(cfg, 42, lengths=[70, 0, 1, 128, 33])
    a = compare(x, label="l2norm varlen", l2=True)
    b = run_bwd(x, use_context=False, l2=True)
    for n, u, v in zip(NAMES, a, b):
        assert np.array_equal(u, v), n


def test_l2norm_metric_shape_fwd_bwd():
    import dataclasses
    cfg = dataclasses.replace(gi.CONFIGS["metric"], name="metric_l2", qk_normalized=False)
    compare(gi.make_inputs(cfg, 0), label="metric shape, raw q/k, in-operator normalisation", l2=True)


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128), ("fp32", 128)])
def test_l2norm_rows_below_the_floor(dtype, d):
    # rows of q and k that are exactly zero lie below the norm floor: the normalised row is
    # zero and its gradient is dy / floor.  Those rows' gradients are ~1e12 times the others',
    # so they are checked on their own and the remaining rows separately.
    cfg = small_cfg(dtype, d, T=150, H=2, with_grad=True, qk_normalized=False)
    x = gi.make_inputs(cfg, 43)
    x["q"] = x["q"].copy()
    x["k"] = x["k"].copy()
    zq, zk = [0, 5, 63, 64, 100], [1, 5, 70, 149]
    x["q"][0, zq, 0] = 0
    x["k"][0, zk, 1] = 0
    say("case", "rows below the floor", dtype, "d", d, "zero q rows (head 0)", zq, "zero k rows (head 1)", zk)
    d_ = dev_inputs(x)
    o, _ = gdn.fwd(d_["q"], d_["k"], d_["v"], d_["g"], d_["beta"], qk_l2norm=True)
    ro, _ = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], qk_l2norm=True)
    o = to_np(o)
    tol = TOL[dtype]
    assert np.all(np.isfinite(o)) and maxrel(o, ro) <= tol["maxrel"], maxrel(o, ro)
    got = run_bwd(x, l2=True)
    ref = ref_bwd(x, l2=True)
    masks = {"dq": (zq, 0), "dk": (zk, 1)}
    for name, a, b in zip(NAMES, got, ref):
        if b is None:
            continue
        assert np.all(np.isfinite(a)), name
        parts = [(a, b)]
        if name in masks:
            rows, h = masks[name]
            sel = np.zeros(a.shape, bool)
            sel[0, rows, h] = True
            assert np.max(np.abs(b[sel])) > 1e6 * np.max(np.abs(b[~sel]))   # the branch was taken
            parts = [(a[sel], b[sel]), (a[~sel], b[~sel])]
        for u, v in parts:
            mr, fr = maxrel(u, v), frob(u, v)
            say("  %-6s maxrel %.3e  frob %.3e" % (name, mr, fr))
            assert mr <= tol["maxrel"] and fr <= tol["frob"], (name, mr, fr)


@pytest.mark.parametrize("dtype,d,B,H", [("fp32", 64, 20, 4), ("bf16", 128, 5, 8), ("bf16", 64, 40, 2),
                                         ("fp32", 128, 5, 8)])
def test_state_passes_grid_past_one_round(dtype, d, B, H):
    # more (sequence, head, 16-column block) workgroups in both state passes
    # than the device has CUs: two column blocks per workgroup, rotated shared reads
    B = batch_past_one_round(B, H, d)
    assert B * H * (d // 16) > device_cus()
    cfg = small_cfg(dtype, d, B=B, T=100, H=H, h0_std=0.05, with_grad=True)
    x = gi.make_inputs(cfg, 41 + d)
    dht = np.random.default_rng(42).standard_normal((B, H, d, d)) * 0.05
    compare(x, dht=dht, scale=0.8, label="state grids past one round")


def test_state_passes_grid_of_one_round_rotated():
    # between half the CU count and the CU count of workgroups: one column block
    # per workgroup, rotated shared reads
    H, d = 8, 128
    B = batch_in_one_round(H, d)
    if B is None:
        pytest.skip("no batch puts this grid between CUs / 2 and CUs")
    assert device_cus() // 2 < B * H * (d // 16) <= device_cus()
    x = gi.make_inputs(small_cfg("bf16", d, B=B, T=130, H=H, h0_std=0.05, with_grad=True), 43)
    dht = np.random.default_rng(44).standard_normal((B, H, d, d)) * 0.05
    compare(x, dht=dht, scale=0.8, label="state grids of one round, rotated")
