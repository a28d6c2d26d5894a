"""GPU: q, k, v given as token-strided views of one [B, T, s] buffer (e.g. a
conv1d output) give bitwise the same results as contiguous copies, in the
forward, the backward (with and without the forward context, the gradients
returned as views of one buffer laid out like the inputs), with in-operator
normalisation, on packed sequences, and in the recurrent forward."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
from gpu_util import dev_inputs, say, small_cfg, to_np

pytestmark = pytest.mark.gpu


def interleave(q, k, v, pad=64):
    """q, k, v [B, T, H, d] -> views of one [B, T, 3*H*d + pad] buffer (and the buffer)."""
    B, T, H, D = q.shape
    w = H * D
    buf = torch.full((B, T, 3 * w + pad), float("nan"), dtype=q.dtype, device=q.device)
    for i, t in enumerate((q, k, v)):
        buf[..., i * w:(i + 1) * w] = t.reshape(B, T, w)
    views = [buf[..., i * w:(i + 1) * w].view(B, T, H, D) for i in range(3)]
    return views, buf


CASES = [("bf16", 128, False, False), ("bf16", 128, True, True), ("fp32", 64, False, True), ("bf16", 64, True, False)]


@pytest.mark.parametrize("dtype,d,l2,packed", CASES)
def test_strided_equals_contiguous(dtype, d, l2, packed):
    cfg = small_cfg(dtype, d, B=1 if packed else 2, T=150, H=2, h0_std=0.1, with_grad=True, qk_normalized=not l2)
    x = gi.make_inputs(cfg, 70, lengths=[40, 0, 1, 109] if packed else None)
    D = dev_inputs(x)
    say("case strided q/k/v", dtype, "d", d, "qk_l2norm", l2, "packed", packed)
    (qs, ks, vs), buf = interleave(D["q"], D["k"], D["v"])
    assert not qs.is_contiguous()
    args = dict(initial_state=D["h0"], cu_seqlens=D["cu"], scale=0.9, qk_l2norm=l2)
    o_c, ht_c, ctx_c = gdn.fwd(D["q"], D["k"], D["v"], D["g"], D["beta"], return_context=True, **args)
    o_s, ht_s, ctx_s = gdn.fwd(qs, ks, vs, D["g"], D["beta"], return_context=True, **args)
    assert torch.equal(o_c, o_s) and torch.equal(ht_c, ht_s)
    g_c = gdn.bwd(D["q"], D["k"], D["v"], D["g"], D["beta"], D["do"], context=ctx_c, **args)
    g_s = gdn.bwd(qs, ks, vs, D["g"], D["beta"], D["do"], context=ctx_s, **args)
    g_r = gdn.bwd(qs, ks, vs, D["g"], D["beta"], D["do"], **args)   # recomputing the forward
    # the gradients come back as views of one buffer laid out like q, k, v
    assert g_s[0].stride() == qs.stride() and g_s[1].untyped_storage().data_ptr() == g_s[0].untyped_storage().data_ptr()
    for a, b, c in zip(g_c, g_s, g_r):
        if a is None:
            continue
        assert torch.equal(a, b) and torch.equal(a, c)
    # the input buffer's padding was never written
    assert torch.isnan(buf[..., 3 * qs.shape[2] * qs.shape[3]:]).all()


def test_strided_recurrent_equals_contiguous():
    N, H, d = 5, 2, 128
    x = gi.make_inputs(small_cfg("bf16", d, B=N, T=2, H=H), 71)
    D = dev_inputs(x)
    (qs, ks, vs), _ = interleave(D["q"], D["k"], D["v"])
    s0 = torch.randn(N, H, d, d, device="cuda") * 0.3
    s_c, s_s = s0.clone(), s0.clone()
    o_c = gdn.recurrent_fwd(D["q"], D["k"], D["v"], D["g"], D["beta"], s_c)
    o_s = gdn.recurrent_fwd(qs, ks, vs, D["g"], D["beta"], s_s)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_s) and torch.equal(s_c, s_s)


def test_conv_output_feeds_the_operator_directly():
    # one conv1d over q, k, v concatenated, the operator on views of its output, and one
    # conv1d backward over the gradients' buffer == three calls per tensor
    T, H, d = 256, 2, 128
    C = 3 * H * d
    cv = gi.make_conv_inputs(1, T, C, 4, "bf16", seed=72)
    x = gi.make_inputs(small_cfg("bf16", d, B=1, T=T, H=H, with_grad=True), 73)
    D = dev_inputs(x)
    xt = torch.from_numpy(cv["x"]).bfloat16().cuda()
    wt = torch.from_numpy(cv["w"]).float().cuda()
    y = gdn.causal_conv1d_fwd(xt, wt)
    q, k, v = (y[..., i * H * d:(i + 1) * H * d].view(1, T, H, d) for i in range(3))
    o, _, ctx = gdn.fwd(q, k, v, D["g"], D["beta"], return_context=True, qk_l2norm=True)
    dq, dk, dv = gdn.bwd(q, k, v, D["g"], D["beta"], D["do"], context=ctx, qk_l2norm=True)[:3]
    dbuf = dq.as_strided((1, T, C), (T * C, C, 1), dq.storage_offset())
    dx, dw, _ = gdn.causal_conv1d_bwd(xt, wt, dbuf)
    # the same through contiguous per-tensor calls
    parts = [xt[..., i * H * d:(i + 1) * H * d].contiguous() for i in range(3)]
    ws = [wt[i * H * d:(i + 1) * H * d].contiguous() for i in range(3)]
    ys = [gdn.causal_conv1d_fwd(p_, w_).view(1, T, H, d) for p_, w_ in zip(parts, ws)]
    o2, _, ctx2 = gdn.fwd(*ys, D["g"], D["beta"], return_context=True, qk_l2norm=True)
    grads = gdn.bwd(*ys, D["g"], D["beta"], D["do"], context=ctx2, qk_l2norm=True)[:3]
    outs = [gdn.causal_conv1d_bwd(p_, w_, g_.view(1, T, H * d)) for p_, w_, g_ in zip(parts, ws, grads)]
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for i in range(3):
        sl = slice(i * H * d, (i + 1) * H * d)
        assert torch.equal(dx[..., sl], outs[i][0]) and torch.equal(dw[sl], outs[i][1])
