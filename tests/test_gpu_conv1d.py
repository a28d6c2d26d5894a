"""GPU parity of the causal depthwise conv1d (HIP path through the C ABI) against
the fp64 oracle (oracle/conv1d.py), element by element on seeded inputs: both
dtypes, K = 1..4, with and without bias and SiLU, ragged channel and token
counts, packed sequences (empty ones, ones shorter than K), the q/k/v
projections of the throughput workload, the packed 32768-token workload, token
counts past the backward's grid rows, and bitwise reproducibility."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
import oracle
from gpu_util import TOL, TORCH_DT, frob, maxrel, say, to_np

pytestmark = pytest.mark.gpu


def dev(a, dt):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()


def run(x, bias=True, act=True):
    dt = TORCH_DT[x["dtype"]]
    xt, dyt = dev(x["x"], dt), dev(x["dy"], dt)
    wt = dev(x["w"], torch.float32)
    bt = dev(x["bias"], torch.float32) if bias else None
    cu = None if x["cu_seqlens"] is None else torch.from_numpy(x["cu_seqlens"])
    y = gdn.causal_conv1d_fwd(xt, wt, bt, cu, act)
    dx, dw, db = gdn.causal_conv1d_bwd(xt, wt, dyt, bt, cu, act)
    torch.cuda.synchronize()
    return [to_np(t) for t in (y, dx, dw, db)]


def ref(x, bias=True, act=True):
    b = x["bias"] if bias else None
    y = oracle.causal_conv1d_fwd(x["x"], x["w"], b, x["cu_seqlens"], act)
    dx, dw, db = oracle.causal_conv1d_bwd(x["x"], x["w"], x["dy"], b, x["cu_seqlens"], act)
    return [y, dx, dw, db]


def check(x, bias=True, act=True, label=""):
    say("case conv1d", label, x["dtype"], "B", x["B"], "T", x["T"], "C", x["C"], "K", x["K"],
        "bias", bias, "act", act, "packed", x["cu_seqlens"] is not None)
    got, want = run(x, bias, act), ref(x, bias, act)
    tol = TOL[x["dtype"]]
    bad = []
    for name, a, b in zip(("y", "dx", "dw", "dbias"), got, want):
        mr, fr = maxrel(a, b), frob(a, b)
        say("  %-5s maxrel %.3e  frob %.3e" % (name, mr, fr))
        if not np.all(np.isfinite(a)):
            bad.append(name + " non-finite")
        elif mr > tol["maxrel"] or fr > tol["frob"]:
            bad.append("%s maxrel %.2e frob %.2e" % (name, mr, fr))
    assert not bad, (label, bad)
    return got


SMALL = [
    ("fp32", 1, 1, 4, 1, True, True), ("fp32", 2, 65, 12, 2, True, False), ("fp32", 1, 200, 260, 3, False, True),
    ("fp32", 2, 63, 64, 4, True, True), ("bf16", 1, 64, 516, 4, True, True), ("bf16", 2, 5, 8, 3, False, False),
    ("bf16", 1, 130, 2048, 4, True, True), ("bf16", 3, 17, 36, 1, True, True), ("bf16", 1, 257, 100, 2, False, True),
]


@pytest.mark.parametrize("dtype,B,T,C,K,bias,act", SMALL)
def test_dense_small(dtype, B, T, C, K, bias, act):
    x = gi.make_conv_inputs(B, T, C, K, dtype, seed=T + C + K)
    check(x, bias, act, "dense")


@pytest.mark.parametrize("dtype,K", [("fp32", 4), ("bf16", 4), ("bf16", 2)])
def test_packed_with_short_and_empty_sequences(dtype, K):
    x = gi.make_conv_inputs(1, 0, 72, K, dtype, seed=7, lengths=[1, 0, 2, 3, 70, 0, 1, 129, 4])
    check(x, True, True, "packed short")


def test_thousands_of_short_sequences():
    # 3000 sequences of 0..9 tokens (more than one planner pass of 1024, many empty): every
    # token's window is clipped by a nearby sequence start or end
    lengths = [int(v) for v in np.random.default_rng(9).integers(0, 10, 3000)]
    x = gi.make_conv_inputs(1, 0, 256, 4, "bf16", seed=9, lengths=lengths)
    check(x, True, True, "3000 short sequences")


def test_throughput_workload_qkv_channels():
    # the short conv of the throughput workload: T = 4096 tokens, q, k, v of 16 heads x 128
    # concatenated (6144 channels), K = 4, SiLU, bf16
    x = gi.make_conv_inputs(1, 4096, 3 * 16 * 128, 4, "bf16", seed=1)
    check(x, True, True, "T4096 C6144")


def test_packed_32768_tokens():
    x = gi.make_conv_inputs(1, 0, 16 * 128, 4, "bf16", seed=2, varlen_total=32768)
    check(x, False, True, "packed 32768 x 2048")


def test_past_the_backward_grid_rows():
    # more token tiles than the backward grid has rows: each workgroup loops
    x = gi.make_conv_inputs(1, 10007, 64, 4, "fp32", seed=3)
    check(x, True, True, "T10007")


def test_bitwise_reproducible():
    x = gi.make_conv_inputs(2, 1000, 256, 4, "bf16", seed=4)
    a, b = run(x), run(x)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_no_tokens_writes_zero_gradients():
    x = torch.empty((1, 0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, 4, device="cuda")
    b = torch.ones(64, device="cuda")
    assert gdn.causal_conv1d_fwd(x, w, b).shape == (1, 0, 64)
    dx, dw, db = gdn.causal_conv1d_bwd(x, w, x, b)
    torch.cuda.synchronize()
    assert torch.all(dw == 0) and torch.all(db == 0)


def test_concatenated_channels_equal_separate_calls():
    # the conv is per channel: one call over q, k, v concatenated (3 x 2048 channels) gives
    # bitwise the same outputs as one call per part (how the operator's q, k, v are fed)
    x = gi.make_conv_inputs(1, 300, 3 * 256, 4, "bf16", seed=8)
    whole = run(x)
    for i in range(3):
        sl = slice(256 * i, 256 * (i + 1))
        part = dict(x, x=np.ascontiguousarray(x["x"][..., sl]), dy=np.ascontiguousarray(x["dy"][..., sl]),
                    w=np.ascontiguousarray(x["w"][sl]), bias=np.ascontiguousarray(x["bias"][sl]), C=256)
        got = run(part)
        assert np.array_equal(got[0], whole[0][..., sl]) and np.array_equal(got[1], whole[1][..., sl])
        assert np.array_equal(got[2], whole[2][sl]) and np.array_equal(got[3], whole[3][sl])
