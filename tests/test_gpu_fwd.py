"""GPU parity of the forward pass (HIP path through the C ABI) against the fp64
oracle, element by element, on seeded inputs."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
import oracle
from gpu_util import batch_past_one_round, check, device_cus, dev_inputs, say, small_cfg, to_np

pytestmark = pytest.mark.gpu


def run_fwd(x, scale=1.0, l2=False):
    d = dev_inputs(x)
    o, ht = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"],
                    cu_seqlens=d["cu"], scale=scale, qk_l2norm=l2)
    torch.cuda.synchronize()
    return to_np(o), to_np(ht)


def ref_fwd(x, scale=1.0, l2=False):
    return oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"],
                      cu_seqlens=x["cu_seqlens"], scale=scale, qk_l2norm=l2)


def compare(x, scale=1.0, label="", l2=False):
    say("case", label, "dtype", x["dtype"], "B", x["B"], "T", x["T"], "H", x["H"], "d", x["dk"],
        "N", x["N"], "qk_l2norm", l2)
    o, ht = run_fwd(x, scale, l2)
    ro, rht = ref_fwd(x, scale, l2)
    check("o", o, ro, x["dtype"], "maxrel")
    if x["dtype"] == "fp32":
        check("ht", ht, rht, "fp32", "maxrel")
    else:
        check("ht", ht, rht, "bf16", "frob")
    return o, ht


def test_config0_fp32():
    compare(gi.make_inputs(gi.CONFIGS["c0"], 0), label="c0")


SMALL = [
    ("fp32", 64, 1, 200, 3, 0.0, 0.7),
    ("fp32", 128, 2, 130, 2, 0.3, 1.0),
    ("fp32", 64, 1, 1, 2, 0.5, 1.0),
    ("bf16", 64, 2, 300, 2, 0.0, 1.0),
    ("bf16", 128, 1, 257, 3, 0.2, 1.0),
    ("bf16", 128, 1, 63, 1, 0.0, 0.125),
    ("bf16", 128, 1, 64, 2, 0.0, 1.0),
    ("bf16", 128, 1, 65, 2, 0.1, 1.0),
]


@pytest.mark.parametrize("dtype,d,B,T,H,h0,scale", SMALL)
def test_small_dense(dtype, d, B, T, H, h0, scale):
    cfg = small_cfg(dtype, d, B=B, T=T, H=H, h0_std=h0)
    compare(gi.make_inputs(cfg, 1), scale=scale, label="small")


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("bf16", 128), ("fp32", 128)])
def test_small_varlen(dtype, d):
    cfg = small_cfg(dtype, d, H=2, h0_std=0.3)
    x = gi.make_inputs(cfg, 2, lengths=[1, 0, 63, 64, 65, 130, 0, 7])
    compare(x, label="varlen")


def test_empty_sequences_pass_state_through():
    cfg = small_cfg("fp32", 64, H=2, h0_std=0.5)
    x = gi.make_inputs(cfg, 3, lengths=[0, 5, 0])
    o, ht = run_fwd(x)
    _, rht = ref_fwd(x)
    assert np.array_equal(ht[0], x["h0"][0]) and np.array_equal(ht[2], x["h0"][2])
    check("ht", ht, rht, "fp32")
    # no tokens at all
    x = gi.make_inputs(cfg, 3, lengths=[0, 0])
    o, ht = run_fwd(x)
    assert o.shape[1] == 0 and np.array_equal(ht, x["h0"])


def test_strong_decay_is_finite():
    cfg = small_cfg("bf16", 128, T=150, H=2)
    x = gi.make_inputs(cfg, 4)
    x["g"] = np.full_like(x["g"], -30.0)
    compare(x, label="g=-30")


def test_bitwise_deterministic():
    cfg = small_cfg("bf16", 128, T=333, H=3, h0_std=0.1)
    x = gi.make_inputs(cfg, 5)
    a = run_fwd(x)
    b = run_fwd(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("name", ["c1", "c2", "c3"])
def test_full_config(name):
    x = gi.make_inputs(gi.CONFIGS[name], 0)
    compare(x, label=name)


# in-operator L2 normalisation of q and k, on raw rows (norms spread over [0.5, 4])
L2 = [
    ("fp32", 64, 1, 200, 2, 0.2, 1.0),
    ("fp32", 128, 1, 130, 2, 0.0, 0.5),
    ("bf16", 64, 2, 150, 2, 0.0, 1.0),
    ("bf16", 128, 1, 257, 3, 0.1, 0.8),
]


@pytest.mark.parametrize("dtype,d,B,T,H,h0,scale", L2)
def test_l2norm_small(dtype, d, B, T, H, h0, scale):
    cfg = small_cfg(dtype, d, B=B, T=T, H=H, h0_std=h0, qk_normalized=False)
    compare(gi.make_inputs(cfg, 31), scale=scale, label="l2norm", l2=True)


def test_l2norm_varlen():
    cfg = small_cfg("bf16", 128, H=2, qk_normalized=False)
    compare(gi.make_inputs(cfg, 32, lengths=[5, 0, 64, 129, 1, 70]), label="l2norm varlen", l2=True)


def test_l2norm_is_a_no_op_on_unit_rows():
    # rows that are already unit length give the plain operator's result up to the rounding
    # of the rescaled rows
    cfg = small_cfg("bf16", 128, T=200, H=2)
    x = gi.make_inputs(cfg, 33)
    a, _ = run_fwd(x)
    b, _ = run_fwd(x, l2=True)
    assert np.max(np.abs(a - b)) <= 2e-2 * np.max(np.abs(a))


@pytest.mark.parametrize("dtype,d,B,H", [("fp32", 64, 20, 4), ("fp32", 128, 5, 8), ("bf16", 128, 5, 8)])
def test_state_pass_grid_past_one_round(dtype, d, B, H):
    # more (sequence, head, 16-column block) workgroups than the device has
    # CUs: the state pass takes two column blocks per workgroup and rotates its
    # shared reads
    B = batch_past_one_round(B, H, d)
    assert B * H * (d // 16) > device_cus()
    x = gi.make_inputs(small_cfg(dtype, d, B=B, T=100, H=H, h0_std=0.05), 31 + d)
    compare(x, scale=0.8, label="state grid past one round")
