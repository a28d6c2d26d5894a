"""The forward and backward captured in a HIP graph (torch.cuda.CUDAGraph, the
library's launches recorded through the C ABI on the capturing stream) and
replayed: nothing in the path allocates, copies, clears memory with a memset
or synchronises, so every replay must reproduce the eager call bit for bit.
The graph is replayed several times with unrelated eager work (another
forward and backward on other inputs, fills) and synchronisations in between,
and each replay's outputs (overwritten with NaN before it) are compared with
the eager ones."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
from gpu_util import dev_inputs, say, small_cfg, to_np

pytestmark = pytest.mark.gpu


def step(d, l2):
    o, ht, ctx = gdn.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["h0"], cu_seqlens=d["cu"],
                         qk_l2norm=l2, return_context=True)
    grads = gdn.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], initial_state=d["h0"], dht=d["dht"],
                    cu_seqlens=d["cu"], context=ctx, qk_l2norm=l2)
    return [o, ht] + list(grads)


def replays_match(x, label, l2=False):
    say("case", label, x["dtype"], "B", x["B"], "T", x["T"], "H", x["H"], "d", x["dk"], "N", x["N"])
    d = dev_inputs(x)
    rng = np.random.default_rng(11)
    d["dht"] = torch.from_numpy(rng.standard_normal((x["N"], x["H"], x["dk"], x["dv"])) * 0.1).float().cuda()
    eager = [to_np(t) for t in step(d, l2)]
    torch.cuda.synchronize()
    # other inputs of the same shape, run eagerly between the replays
    y = dev_inputs(gi.make_inputs(small_cfg(x["dtype"], x["dk"], H=x["H"], with_grad=True), 5, T=x["T"], B=x["B"],
                                  lengths=None if x["cu_seqlens"] is None else list(np.diff(x["cu_seqlens"]))))
    y["dht"] = d["dht"] * 2
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step(d, l2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step(d, l2)
    junk = torch.empty(1 << 22, dtype=torch.float32, device="cuda")
    for rep in range(4):
        other = step(y, l2)          # eager work on other inputs between replays
        junk.fill_(float(rep + 1))
        for t in outs:               # the replay must write every output again
            if t is not None:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outs)):
            if a is None:
                assert b is None
                continue
            assert np.array_equal(a, to_np(b)), "replay %d: output %d differs from the eager call" % (rep, i)
        del other


def test_dense_bf16_fwd_bwd_graph_replays():
    cfg = small_cfg("bf16", 128, H=4, h0_std=0.1, with_grad=True)
    x = gi.make_inputs(cfg, 3, T=1000)
    replays_match(x, "dense bf16 T=1000 H=4 d=128 with h0 and dht")


def test_packed_fp32_fwd_bwd_graph_replays_with_l2norm():
    cfg = small_cfg("fp32", 64, H=2, h0_std=0.3, with_grad=True, qk_normalized=False)
    x = gi.make_inputs(cfg, 4, lengths=[1, 0, 63, 64, 65, 130])
    replays_match(x, "packed fp32 d=64, qk_l2norm", l2=True)
