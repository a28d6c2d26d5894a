"""The allocation-free forward (gdn_fwd_noalloc, workspace in the library's
static per-GPU scratch) against gdn_fwd with a caller workspace: the same
kernels, so o and ht must agree bit for bit, on two calls in a row, the
second smaller than the first (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
import oracle
from gpu_util import check, dev_inputs, say, small_cfg, to_np

pytestmark = pytest.mark.gpu


def both(x, scale=1.0, l2=False):
    d = dev_inputs(x)
    a = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"], cu_seqlens=d["cu"],
                scale=scale, qk_l2norm=l2)
    b = gdn.fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"], cu_seqlens=d["cu"],
                        scale=scale, qk_l2norm=l2)
    torch.cuda.synchronize()
    return [to_np(t) for t in a], [to_np(t) for t in b]


def agree(x, label, scale=1.0, l2=False):
    say("case", label, x["dtype"], "B", x["B"], "T", x["T"], "H", x["H"], "d", x["dk"], "N", x["N"])
    (o, ht), (o2, ht2) = both(x, scale, l2)
    assert np.array_equal(o, o2), "o differs from gdn_fwd"
    assert np.array_equal(ht, ht2), "ht differs from gdn_fwd"
    return o2, ht2


def test_two_calls_second_smaller():
    # the throughput workload's forward (it fits the 128 MiB scratch), then a small packed one
    x = gi.make_inputs(gi.CONFIGS["c1"], 0)
    agree(x, "T=4096 H=16 d=128 bf16")
    cfg = small_cfg("fp32", 64, H=2, h0_std=0.3)
    x = gi.make_inputs(cfg, 2, lengths=[1, 0, 63, 64, 65, 130, 0, 7])
    o, ht = agree(x, "packed fp32 d=64 with h0", scale=0.7)
    ro, rht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], cu_seqlens=x["cu_seqlens"], scale=0.7)
    check("o", o, ro, "fp32")
    check("ht", ht, rht, "fp32")


def test_two_calls_normalised_then_smaller():
    cfg = small_cfg("bf16", 128, B=2, T=700, H=3, h0_std=0.1, qk_normalized=False)
    agree(gi.make_inputs(cfg, 3), "bf16 d=128 in-operator normalisation", l2=True)
    cfg = small_cfg("bf16", 128, T=65, H=1)
    x = gi.make_inputs(cfg, 4)
    o, ht = agree(x, "bf16 d=128 T=65")
    ro, rht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    check("o", o, ro, "bf16")
    check("ht", ht, rht, "bf16", "frob")


def test_preallocated_outputs_and_too_large_problem():
    x = gi.make_inputs(small_cfg("bf16", 64, T=300, H=2), 5)
    d = dev_inputs(x)
    o = torch.empty_like(d["v"])
    ht = torch.empty((1, 2, 64, 64), dtype=torch.float32, device=o.device)
    r = gdn.fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], out=o, final_state=ht)
    assert r[0].data_ptr() == o.data_ptr() and r[1].data_ptr() == ht.data_ptr()
    ref = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(ht, ref[1])
    # beyond the static scratch: rejected before anything is enqueued
    q = torch.zeros((1, 8192, 16, 128), dtype=torch.bfloat16, device=o.device)
    g = torch.zeros((1, 8192, 16), dtype=torch.float32, device=o.device)
    with pytest.raises(gdn.GdnError) as e:
        gdn.fwd_noalloc(q, q, q, g, g)
    assert e.value.status == gdn.GDN_ERR_UNSUPPORTED
