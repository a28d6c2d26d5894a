"""GPU: a dense bf16 problem whose q, k, v, o and gradient tensors pass 2^31 elements
(272 sequences x 4096 tokens x 16 heads x 128; the element offsets of sequences 256 and up
need 64-bit arithmetic), forward with h0 and backward with dht and dh0, compared with the fp64
oracle on sampled sequences on both sides of that boundary.  About 135 GB of device memory."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
import oracle
from gpu_util import TOL, frob, maxrel, say

pytestmark = pytest.mark.gpu

B, T, H, D = 272, 4096, 16, 128
SAMPLED = (0, 255, 256, 271)


def host(t, n):
    return t[n:n + 1].to(torch.float64).cpu().numpy()


def test_tensors_past_2_31_elements():
    assert B * T * H * D > 2 ** 31 and (B - 16) * T * H * D == 2 ** 31   # sequence 256 starts at 2^31
    torch.cuda.empty_cache()   # memory cached by earlier tests of this process
    free, _ = torch.cuda.mem_get_info()
    if free < 160 * 2 ** 30:
        pytest.skip("needs about 135 GB of free device memory (%.0f GB free)" % (free / 2 ** 30))
    x = gi.make_inputs_device(B, T, H, D, seed=90, device="cuda")
    say("case large dense B", B, "T", T, "H", H, "d", D, "elements per tensor", B * T * H * D)
    o, ht, ctx = gdn.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], initial_state=x["h0"], return_context=True)
    grads = gdn.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], initial_state=x["h0"], dht=x["dht"],
                    context=ctx)
    torch.cuda.synchronize()
    del ctx
    tol = TOL["bf16"]
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    for n in SAMPLED:
        xs = {k_: host(v_, n) for k_, v_ in x.items()}
        ro, rht = oracle.fwd(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"])
        rg = oracle.bwd(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["do"], xs["h0"], xs["dht"])
        got_o, got_ht = host(o, n), host(ht, n)
        say("  seq %d: o maxrel %.3e  ht frob %.3e" % (n, maxrel(got_o, ro), frob(got_ht, rht)))
        assert np.all(np.isfinite(got_o)) and maxrel(got_o, ro) <= tol["maxrel"], n
        assert frob(got_ht, rht) <= tol["frob"], n
        for nm, a, b in zip(names, grads, rg):
            got = host(a, n)
            mr, fr = maxrel(got, b), frob(got, b)
            say("    %-6s maxrel %.3e  frob %.3e" % (nm, mr, fr))
            assert np.all(np.isfinite(got)) and mr <= tol["maxrel"] and fr <= tol["frob"], (n, nm, mr, fr)
    del x, o, ht, grads
    torch.cuda.empty_cache()   # hand the memory back for the tests after this one
