"""GPU parity of the gated RMSNorm on the operator's output (HIP path through the
C ABI) against the fp64 oracle (oracle/gated_norm.py), element by element on
seeded inputs: both dtypes and row lengths, ragged row counts, a row count
past the backward's workgroup cap (grid-stride rounds), the operator-output
shape of the throughput workload, zero rows, saturated gates, no rows, and
bitwise reproducibility."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
import oracle
from gpu_util import TOL, TORCH_DT, frob, maxrel, say, to_np

pytestmark = pytest.mark.gpu


def dev(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()


def run(x, eps):
    dt = TORCH_DT[x["dtype"]]
    xt, zt, dyt = (dev(x[n], dt) for n in ("x", "z", "dy"))
    wt = dev(x["w"], torch.float32)
    y = gdn.gated_rmsnorm_fwd(xt, zt, wt, eps)
    dx, dz, dw = gdn.gated_rmsnorm_bwd(xt, zt, wt, dyt, eps)
    torch.cuda.synchronize()
    return [to_np(t) for t in (y, dx, dz, dw)]


def ref(x, eps):
    y = oracle.gated_rmsnorm_fwd(x["x"], x["z"], x["w"], eps)
    dx, dz, dw = oracle.gated_rmsnorm_bwd(x["x"], x["z"], x["w"], x["dy"], eps)
    return [y, dx, dz, dw]


def check(got, want, dtype, label):
    tol = TOL[dtype]
    bad = []
    for name, a, b in zip(("y", "dx", "dz", "dw"), got, want):
        mr, fr = maxrel(a, b), frob(a, b)
        say("  %-3s %-24s maxrel %.3e  frob %.3e" % (name, label, mr, fr))
        if not np.all(np.isfinite(a)):
            bad.append(name + " non-finite")
        elif mr > tol["maxrel"] or fr > tol["frob"]:
            bad.append("%s maxrel %.2e frob %.2e" % (name, mr, fr))
    assert not bad, (label, bad)


CASES = [
    ("fp32", 64, 1, 1e-6), ("fp32", 64, 257, 1e-6), ("fp32", 128, 1000, 1e-2),
    ("bf16", 64, 3, 1e-6), ("bf16", 64, 4099, 1e-6), ("bf16", 128, 63, 1e-6),
    ("bf16", 128, 1025, 1e-5), ("fp32", 128, 4097, 1e-6),
]


@pytest.mark.parametrize("dtype,dim,rows,eps", CASES)
def test_small(dtype, dim, rows, eps):
    say("case gated norm", dtype, "dim", dim, "rows", rows, "eps", eps)
    x = gi.make_gated_norm_inputs(rows, dim, dtype, seed=rows + dim)
    check(run(x, eps), ref(x, eps), dtype, "%s d%d rows%d" % (dtype, dim, rows))


@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("fp32", 64)])
def test_past_the_backward_workgroup_cap(dtype, dim):
    # more row pieces than the capped backward grid covers in one round
    rows = 200_003
    say("case gated norm", dtype, "dim", dim, "rows", rows)
    x = gi.make_gated_norm_inputs(rows, dim, dtype, seed=11)
    check(run(x, 1e-6), ref(x, 1e-6), dtype, "%s d%d rows%d" % (dtype, dim, rows))


def test_on_the_operator_output_of_the_throughput_workload():
    # x = the operator's output o at B=1, T=4096, H=16, d=128 (bf16), computed by the HIP path
    cfg = gi.CONFIGS["metric"]
    g = gi.make_inputs(cfg, 0)
    say("case gated norm on o of", cfg.name)
    d = {n: dev(g[n], torch.bfloat16) for n in ("q", "k", "v")}
    o, _ = gdn.fwd(d["q"], d["k"], d["v"], dev(g["g"], torch.float32), dev(g["beta"], torch.float32))
    rows = cfg.B * cfg.T * cfg.H
    x = gi.make_gated_norm_inputs(rows, 128, "bf16", seed=5, x=to_np(o))
    check(run(x, 1e-6), ref(x, 1e-6), "bf16", "metric-shape o")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_zero_rows_and_saturated_gates(dtype):
    # zero rows: y = 0 and dx = dn / sqrt(eps), about 1e3 times the other rows' gradients,
    # so dx is checked on those rows and on the rest separately; gates of +-30 and +-90
    # saturate the sigmoid
    rows, dim, eps = 300, 128, 1e-6
    x = gi.make_gated_norm_inputs(rows, dim, dtype, seed=3)
    zero = np.zeros(rows, bool)
    zero[[0, 7, 150, 299]] = True
    x["x"] = x["x"].copy()
    x["x"][zero] = 0.0
    x["z"] = x["z"].copy()
    x["z"][10:20] = 30.0
    x["z"][20:30] = -30.0
    x["z"][30:40, ::2] = 90.0
    x["z"][30:40, 1::2] = -90.0
    say("case gated norm zero rows / saturated gates", dtype)
    got, want = run(x, eps), ref(x, eps)
    assert np.all(got[0][zero] == 0)
    check([got[0], got[1][~zero], got[2], got[3]], [want[0], want[1][~zero], want[2], want[3]],
          dtype, "%s other rows" % dtype)
    mr, fr = maxrel(got[1][zero], want[1][zero]), frob(got[1][zero], want[1][zero])
    say("  dx  zero rows               maxrel %.3e  frob %.3e" % (mr, fr))
    assert mr <= TOL[dtype]["maxrel"] and fr <= TOL[dtype]["frob"]


def test_no_rows_writes_zero_dw():
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(128, device="cuda")
    assert gdn.gated_rmsnorm_fwd(x, x, w).shape == (0, 128)
    dx, dz, dw = gdn.gated_rmsnorm_bwd(x, x, w, x)
    torch.cuda.synchronize()
    assert dx.shape == (0, 128) and dz.shape == (0, 128)
    assert torch.all(dw == 0)


def test_bitwise_reproducible_and_layout_free_of_shape():
    x = gi.make_gated_norm_inputs(5000, 128, "bf16", seed=9)
    a = run(x, 1e-6)
    b = run(x, 1e-6)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    # a [B, T, H, d] view gives the same result as the flat rows
    dt = torch.bfloat16
    xt, zt, dyt = (dev(x[n], dt) for n in ("x", "z", "dy"))
    wt = dev(x["w"], torch.float32)
    y4 = gdn.gated_rmsnorm_fwd(xt.view(2, 125, 20, 128), zt.view(2, 125, 20, 128), wt)
    assert np.array_equal(to_np(y4).reshape(5000, 128), a[0])
