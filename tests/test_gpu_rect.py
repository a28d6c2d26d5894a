"""GPU parity of the chunked forward and backward with d_k != d_v (64 and 128
either way) against the fp64 oracle, which runs the token recurrence on the
rectangular d_v x d_k state as it is.  The kernels run at the larger head dim
with the narrower tensor read as zeros past its width; the tests also check
that nothing past the real widths is written."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
from gpu_util import dev_inputs, say, small_cfg
from test_gpu_bwd import NAMES, compare as compare_bwd, run_bwd
from test_gpu_fwd import compare as compare_fwd

pytestmark = pytest.mark.gpu

RECT_FWD = [
    ("fp32", 64, 128, 1, 200, 2, 0.2, 0.8),
    ("fp32", 128, 64, 2, 130, 2, 0.0, 1.0),
    ("bf16", 64, 128, 1, 300, 3, 0.1, 1.0),
    ("bf16", 128, 64, 1, 257, 2, 0.1, 0.5),
    ("bf16", 128, 64, 1, 1, 1, 0.3, 1.0),
]


@pytest.mark.parametrize("dtype,dk,dv,B,T,H,h0,scale", RECT_FWD)
def test_rect_forward(dtype, dk, dv, B, T, H, h0, scale):
    cfg = small_cfg(dtype, 64, dk=dk, dv=dv, B=B, T=T, H=H, h0_std=h0)
    compare_fwd(gi.make_inputs(cfg, 81), scale=scale, label="dk=%d dv=%d" % (dk, dv))


RECT_BWD = [
    ("fp32", 64, 128, 1, 200, 2, 0.2, True, 0.8),
    ("fp32", 128, 64, 2, 130, 1, 0.0, False, 1.0),
    ("bf16", 64, 128, 2, 300, 2, 0.1, True, 1.0),
    ("bf16", 128, 64, 1, 257, 3, 0.0, True, 1.0),
]


@pytest.mark.parametrize("dtype,dk,dv,B,T,H,h0,with_dht,scale", RECT_BWD)
def test_rect_backward(dtype, dk, dv, B, T, H, h0, with_dht, scale):
    cfg = small_cfg(dtype, 64, dk=dk, dv=dv, B=B, T=T, H=H, h0_std=h0, with_grad=True)
    x = gi.make_inputs(cfg, 82)
    dht = np.random.default_rng(83).standard_normal((x["N"], H, dk, dv)) * 0.1 if with_dht else None
    got = compare_bwd(x, dht=dht, scale=scale, label="dk=%d dv=%d" % (dk, dv))
    assert got[0].shape[-1] == dk and got[1].shape[-1] == dk and got[2].shape[-1] == dv
    assert got[5].shape[-2:] == (dk, dv)
    # the saved forward context and the recomputed one give the same bits
    again = run_bwd(x, dht=dht, scale=scale, use_context=False)
    for n, a, b in zip(NAMES, got, again):
        assert np.array_equal(a, b), n


@pytest.mark.parametrize("dtype,dk,dv", [("fp32", 64, 128), ("bf16", 128, 64), ("bf16", 64, 128)])
def test_rect_packed_fwd_bwd(dtype, dk, dv):
    cfg = small_cfg(dtype, 64, dk=dk, dv=dv, H=2, h0_std=0.2, with_grad=True)
    x = gi.make_inputs(cfg, 84, lengths=[1, 0, 63, 64, 65, 130, 0, 7])
    dht = np.random.default_rng(85).standard_normal((x["N"], 2, dk, dv)) * 0.1
    compare_fwd(x, label="packed dk=%d dv=%d" % (dk, dv))
    got = compare_bwd(x, dht=dht, label="packed dk=%d dv=%d" % (dk, dv))
    # empty sequences pass the state and its gradient through
    assert np.array_equal(got[5][1], dht[1].astype(np.float32))


@pytest.mark.parametrize("dtype,dk,dv", [("fp32", 128, 64), ("bf16", 64, 128)])
def test_rect_l2norm(dtype, dk, dv):
    cfg = small_cfg(dtype, 64, dk=dk, dv=dv, T=190, H=2, h0_std=0.1, with_grad=True, qk_normalized=False)
    x = gi.make_inputs(cfg, 86)
    compare_fwd(x, label="l2norm dk=%d dv=%d" % (dk, dv), l2=True)
    compare_bwd(x, label="l2norm dk=%d dv=%d" % (dk, dv), l2=True)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 64, 128), ("fp32", 128, 64)])
def test_rect_strided_and_no_write_past_the_widths(dtype, dk, dv):
    # q, k, v as token-strided views of one buffer whose other columns hold NaN: the results
    # equal the contiguous ones bit for bit, and the gradients land only in their own columns
    B, T, H = 2, 150, 2
    x = gi.make_inputs(small_cfg(dtype, 64, dk=dk, dv=dv, B=B, T=T, H=H, h0_std=0.1, with_grad=True), 87)
    D = dev_inputs(x)
    wq, wv = H * dk, H * dv
    S = 2 * wq + wv + 64
    buf = torch.full((B, T, S), float("nan"), dtype=D["q"].dtype, device=D["q"].device)
    buf[..., :wq] = D["q"].reshape(B, T, wq)
    buf[..., wq:2 * wq] = D["k"].reshape(B, T, wq)
    buf[..., 2 * wq:2 * wq + wv] = D["v"].reshape(B, T, wv)
    qs = buf[..., :wq].view(B, T, H, dk)
    ks = buf[..., wq:2 * wq].view(B, T, H, dk)
    vs = buf[..., 2 * wq:2 * wq + wv].view(B, T, H, dv)
    say("case strided dk", dk, "dv", dv, dtype)
    a = dict(initial_state=D["h0"], scale=0.9)
    o_c, ht_c, ctx_c = gdn.fwd(D["q"], D["k"], D["v"], D["g"], D["beta"], return_context=True, **a)
    o_s, ht_s, ctx_s = gdn.fwd(qs, ks, vs, D["g"], D["beta"], return_context=True, **a)
    g_c = gdn.bwd(D["q"], D["k"], D["v"], D["g"], D["beta"], D["do"], context=ctx_c, **a)
    g_s = gdn.bwd(qs, ks, vs, D["g"], D["beta"], D["do"], context=ctx_s, **a)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_s) and torch.equal(ht_c, ht_s)
    for u, v in zip(g_c, g_s):
        assert torch.equal(u, v)
    # the gradient buffer (laid out like the inputs) was written only in the q, k, v columns
    gbuf = g_s[0].as_strided((B, T, S), (T * S, S, 1), g_s[0].storage_offset())
    assert torch.isfinite(gbuf[..., :2 * wq + wv]).all()
    assert torch.isnan(buf[..., 2 * wq + wv:]).all()


def test_rect_states_untouched_past_their_size():
    # ht and dh0 are [N, H, dk, dv]: sentinels right after them in one allocation stay intact
    dk, dv, H = 64, 128, 2
    x = gi.make_inputs(small_cfg("bf16", 64, dk=dk, dv=dv, T=100, H=H, h0_std=0.1, with_grad=True), 88)
    D = dev_inputs(x)
    n = H * dk * dv
    store = torch.full((2 * n + 1024,), 7.0, dtype=torch.float32, device="cuda")
    ht = store[:n].view(1, H, dk, dv)
    o, _ = gdn.fwd_noalloc(D["q"], D["k"], D["v"], D["g"], D["beta"], initial_state=D["h0"], final_state=ht)
    o2, ht2 = gdn.fwd(D["q"], D["k"], D["v"], D["g"], D["beta"], initial_state=D["h0"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ht, ht2)
    assert (store[n:] == 7.0).all()
