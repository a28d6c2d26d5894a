"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer:

- the fp64 oracle (oracle/gdn_oracle.c) in a small driver, on packed
  sequences with empty ones, d_k != d_v, h0 and dht, several threads; its
  outputs must equal the regular build's bit for bit;
- the host side of libgdn's C ABI (argument validation, the strided-overlap
  arithmetic, the workspace layout) with the kernel launchers replaced by
  stubs that abort if reached; every call in the driver must be rejected.

Any sanitizer report makes the program exit non-zero (halt_on_error)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import gdn_inputs as gi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_address_and_ub_sanitizers(tmp_path, oracle_mod):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c11", "-pthread", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", exe, "-lm"])
    cfg = gi.Config("san", 1, 1, 2, 8, 5, "fp32", h0_std=0.3, with_grad=True)
    x = gi.make_inputs(cfg, 91, lengths=[0, 7, 1, 0, 70, 64, 3])
    dht = np.random.default_rng(92).standard_normal((x["N"], 2, 8, 5)) * 0.2
    N, H, T = x["N"], x["H"], x["T"]
    inp = str(tmp_path / "in.bin")
    with open(inp, "wb") as f:
        np.array([N, H, 8, 5, T, 1, 1, 3], np.int64).tofile(f)
        np.array([0.8], np.float64).tofile(f)
        x["cu_seqlens"].astype(np.int64).tofile(f)
        for a in (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["do"], dht):
            np.ascontiguousarray(a, np.float64).tofile(f)
    out = str(tmp_path / "out.bin")
    r = _run([exe, inp, out], env=SAN_ENV)
    assert "ok" in r.stdout
    got = np.fromfile(out, np.float64)
    o, ht = oracle_mod.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], cu_seqlens=x["cu_seqlens"], scale=0.8)
    grads = oracle_mod.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], x["h0"], dht,
                           cu_seqlens=x["cu_seqlens"], scale=0.8)
    ref = np.concatenate([a.ravel() for a in (o, ht) + tuple(grads)])
    assert got.shape == ref.shape and np.array_equal(got, ref)


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_abi_host_side_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_asan")
    csrc = os.path.join(ROOT, "linear_attention_gated_amd", "csrc")
    # host code only is instrumented (each -fsanitize= after -Xarch_host); the device side
    # of api.cpp (the static scratch array) is compiled as usual
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=undefined",
          "-x", "hip", os.path.join(csrc, "api.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
          os.path.join(HERE, "abi_driver.cpp"), "-o", exe], timeout=600)
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert r.stdout.startswith("ok ") and int(r.stdout.split()[1]) > 400, r.stdout
