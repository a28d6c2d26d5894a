"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
call the HIP path through the C ABI, and compare with the fp64 oracle."""
import sys

import numpy as np
import torch

import gdn_inputs as gi

TORCH_DT = {"bf16": torch.bfloat16, "fp32": torch.float32}

# Tolerances: fp32 path max relative error 1e-4; bf16 path
# max|o - o_ref| / max|o_ref| <= 2e-2 and relative Frobenius error of the
# final state <= 1e-2 (the same pair is applied to every gradient).
TOL = {"fp32": dict(maxrel=1e-4, frob=1e-4), "bf16": dict(maxrel=2e-2, frob=1e-2)}


def device_cus():
    """Compute units of the current device: the state passes pick their
    instance (one or two column blocks per workgroup, rotated reads) from the
    ratio of their workgroup count to this."""
    return torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count


def batch_past_one_round(B, H, d):
    """The smallest batch >= B whose state-pass grid, B * H * (d / 16)
    workgroups, exceeds the device's compute units."""
    return max(B, device_cus() // (H * (d // 16)) + 1)


def batch_in_one_round(H, d):
    """A batch whose state-pass grid lies in (CUs / 2, CUs], or None."""
    per, cus = H * (d // 16), device_cus()
    B = cus // per
    return B if B >= 1 and cus // 2 < B * per <= cus else None


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def maxrel(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(x)))
    return float(np.max(np.abs(x - ref)) / den)


def frob(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    if den == 0:
        return float(np.linalg.norm(x))
    return float(np.linalg.norm(x - ref) / den)


def dev_inputs(x, device="cuda"):
    """Torch device tensors holding exactly the generator's rounded values."""
    dt = TORCH_DT[x["dtype"]]

    def t(a, d):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(d).to(device)

    out = dict(q=t(x["q"], dt), k=t(x["k"], dt), v=t(x["v"], dt), g=t(x["g"], torch.float32),
               beta=t(x["beta"], torch.float32), h0=t(x["h0"], torch.float32),
               do=t(x["do"], dt))
    cu = x["cu_seqlens"]
    out["cu"] = None if cu is None else (torch.from_numpy(cu).to(torch.int32),
                                         torch.from_numpy(cu).to(torch.int32).to(device))
    return out


def to_np(t):
    return None if t is None else t.detach().to(torch.float64).cpu().numpy()


def check(name, x, ref, dtype, kind="maxrel"):
    tol = TOL[dtype][kind]
    err = maxrel(x, ref) if kind == "maxrel" else frob(x, ref)
    say("  %-6s %s = %.3e (tol %.0e)" % (name, kind, err, tol))
    assert np.all(np.isfinite(x)), name + " has non-finite values"
    assert err <= tol, "%s %s %.3e > %.0e" % (name, kind, err, tol)
    return err


def small_cfg(dtype, d, **kw):
    base = dict(name="small", B=1, T=64, H=2, dk=d, dv=d, dtype=dtype)
    base.update(kw)
    return gi.Config(**base)
