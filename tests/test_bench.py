"""The benchmark's accounting, checked on the CPU: the per-kernel flops and the
operator's bytes add up to the chunked algorithm's totals, the HBM-traffic
summary is read only when it matches the kernel sources, and a request for
more than one GPU is refused before anything touches a GPU."""
import os
import subprocess
import sys

import bench

C, D = 64, 128


def test_kernel_flops_sum_to_the_chunked_algorithm():
    # forward 5 C^2 D + 6 C D^2 + C^3 / 3 and backward 12 C^2 D + 12 C D^2 + 2 C^3 / 3
    # per chunk (2mnk per product, triangular operands at one half): 438,272 flop
    # per token and head at C = 64, D = 128
    from fractions import Fraction
    fl = bench.kernel_flops(D, 1)
    fwd = Fraction(5 * C * C * D + 6 * C * D * D) + Fraction(C ** 3, 3)
    bwd = Fraction(12 * C * C * D + 12 * C * D * D) + Fraction(2 * C ** 3, 3)
    # the per-kernel counts are integers: the C^3 / 3 terms rounded down
    assert abs(fl["fwd_prep"] + fl["fwd_state"] + fl["fwd_out"] - fwd) < 1
    assert abs(fl["bwd_prep"] + fl["bwd_state"] + fl["bwd_grad"] - bwd) < 1
    assert (fwd + bwd) / C == 438272


def test_operator_bytes_per_token_and_head():
    # bf16: the forward reads q, k, v, g, beta and writes o (1,032 B); the backward reads
    # q, k, v, dO, g, beta and writes dq, dk, dv, dg, dbeta (1,808 B, all in bwd_grad)
    _, per_unit = bench.op_bytes(D, 2, 1, 0, with_ht=False)
    assert per_unit["bwd_grad"] // C == 1808
    # k is read by both forward kernels, so their sum counts it twice
    assert (per_unit["fwd_prep"] + per_unit["fwd_out"]) // C == 1032 + 2 * D
    assert per_unit["bwd_prep"] == per_unit["bwd_state"] == per_unit["fwd_state"] == 0


def test_traffic_summary_read_only_at_matching_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    body = "traffic bwd_grad fetch_bytes 100 write_bytes 23\n"
    (tmp_path / "profiles" / "t.txt").write_text("sources_sha %s\n%s" % (bench.sources_sha(), body))
    (tmp_path / "profiles" / "stale.txt").write_text("sources_sha 0000000000000000\n" + body)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_sha", lambda: open(tmp_path / "profiles" / "t.txt").read().split()[1])
    assert bench.traffic_for("bwd_grad", "t.txt") == 123
    assert bench.traffic_for("fwd_out", "t.txt") is None
    assert bench.traffic_for("bwd_grad", "stale.txt") is None
    assert bench.traffic_for("bwd_grad", "missing.txt") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
