"""GPU parity of the recurrent (decoding) forward (HIP path through the C ABI)
against the fp64 oracle's token loop, on seeded inputs: every (d_k, d_v) pair,
both dtypes, in-operator normalisation, state slots with skipped and
out-of-range indices, packed sequences, one call of T tokens against T calls
of one token (bitwise), a chunked prefill followed by decoding, and a long
single call."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
import linear_attention_gated_amd as gdn
import oracle
from gpu_util import TOL, dev_inputs, frob, maxrel, say, small_cfg, to_np

pytestmark = pytest.mark.gpu


def run_rec(x, state, idx=None, scale=1.0, l2=False):
    d = dev_inputs(x)
    st = torch.from_numpy(np.ascontiguousarray(state)).float().cuda()
    it = None if idx is None else torch.tensor(idx, dtype=torch.int32, device="cuda")
    o = gdn.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, it, d["cu"], scale, l2)
    torch.cuda.synchronize()
    return to_np(o), st.cpu().numpy().astype(np.float64)


def check_pair(name, got, want, dtype, kind):
    mr, fr = maxrel(got, want), frob(got, want)
    say("  %-6s maxrel %.3e  frob %.3e" % (name, mr, fr))
    tol = TOL[dtype]
    assert np.all(np.isfinite(got)), name
    if kind == "maxrel":
        assert mr <= tol["maxrel"], (name, mr)
    else:
        assert fr <= tol["frob"] and (dtype == "bf16" or mr <= tol["maxrel"]), (name, mr, fr)


def initial_state(N, H, dk, dv, seed, std=0.5):
    return np.random.default_rng(seed).standard_normal((N, H, dk, dv)) * std


CASES = [(dt, dk, dv, T, l2) for dt in ("fp32", "bf16") for dk in (64, 128) for dv in (64, 128)
         for T, l2 in ((1, False), (3, True))]


@pytest.mark.parametrize("dtype,dk,dv,T,l2", CASES)
def test_decode_against_oracle(dtype, dk, dv, T, l2):
    N, H = 6, 3
    cfg = small_cfg(dtype, dk, dv=dv, B=N, T=T, H=H, qk_normalized=not l2)
    x = gi.make_inputs(cfg, 50 + dk + dv + T)
    s0 = initial_state(N, H, dk, dv, 1)
    say("case recurrent", dtype, "dk", dk, "dv", dv, "N", N, "T", T, "H", H, "qk_l2norm", l2)
    o, st = run_rec(x, s0, scale=0.7, l2=l2)
    ro, rht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, scale=0.7, qk_l2norm=l2)
    check_pair("o", o, ro, dtype, "maxrel")
    check_pair("state", st, rht, dtype, "frob")


def test_state_slots_skips_and_untouched_slots():
    N, H, d, slots = 6, 2, 128, 9
    cfg = small_cfg("bf16", d, B=N, T=2, H=H)
    x = gi.make_inputs(cfg, 61)
    pool = initial_state(slots, H, d, d, 2)
    idx = [7, 2, -1, 5, 9, 0]        # -1 and 9 (== slots) name no slot: those sequences are skipped
    say("case recurrent slots", idx)
    o, st = run_rec(x, pool, idx)
    live = [n for n, s in enumerate(idx) if 0 <= s < slots]
    used = [idx[n] for n in live]
    ro, rht = oracle.fwd(x["q"][live], x["k"][live], x["v"][live], x["g"][live], x["beta"][live], pool[used])
    check_pair("o", o[live], ro, "bf16", "maxrel")
    check_pair("state", st[used], rht, "bf16", "frob")
    for n, s in enumerate(idx):
        if not 0 <= s < slots:
            assert np.all(o[n] == 0), n
    pool32 = pool.astype(np.float32).astype(np.float64)
    for s in range(slots):
        if s not in used:
            assert np.array_equal(st[s], pool32[s]), s


def test_packed_sequences():
    cfg = small_cfg("bf16", 128, H=2)
    x = gi.make_inputs(cfg, 62, lengths=[1, 0, 3, 2, 5])
    N = 5
    s0 = initial_state(N, 2, 128, 128, 3)
    say("case recurrent packed", [1, 0, 3, 2, 5])
    o, st = run_rec(x, s0)
    ro, rht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, cu_seqlens=x["cu_seqlens"])
    check_pair("o", o, ro, "bf16", "maxrel")
    check_pair("state", st, rht, "bf16", "frob")


def test_thousands_of_sequences():
    lengths = [int(v) for v in np.random.default_rng(66).integers(0, 4, 3000)]
    cfg = small_cfg("bf16", 64, H=2)
    x = gi.make_inputs(cfg, 67, lengths=lengths)
    s0 = initial_state(x["N"], 2, 64, 64, 6, std=0.2)
    say("case recurrent 3000 packed sequences")
    o, st = run_rec(x, s0)
    ro, rht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0, cu_seqlens=x["cu_seqlens"])
    check_pair("o", o, ro, "bf16", "maxrel")
    check_pair("state", st, rht, "bf16", "frob")


@pytest.mark.parametrize("dtype,d,l2", [("fp32", 64, False), ("bf16", 128, True)])
def test_one_call_equals_token_by_token_calls(dtype, d, l2):
    # d = 128 spreads a head's state over four waves (sums across waves in LDS)
    N, H, T = 4, 2, 5
    x = gi.make_inputs(small_cfg(dtype, d, B=N, T=T, H=H, qk_normalized=not l2), 63 + d)
    s0 = initial_state(N, H, d, d, 4)
    say("case recurrent token by token", dtype, "d", d, "qk_l2norm", l2)
    o_all, st_all = run_rec(x, s0, l2=l2)
    st = s0.copy()
    for t in range(T):
        xt = dict(x, q=x["q"][:, t:t + 1], k=x["k"][:, t:t + 1], v=x["v"][:, t:t + 1], g=x["g"][:, t:t + 1],
                  beta=x["beta"][:, t:t + 1], do=None, h0=None)
        o_t, st = run_rec(xt, st, l2=l2)
        assert np.array_equal(o_t[:, 0], o_all[:, t]), t
    assert np.array_equal(st, st_all)


def test_repeated_calls_are_bitwise_equal():
    N, H, T, d = 8, 4, 3, 128
    x = gi.make_inputs(small_cfg("bf16", d, B=N, T=T, H=H, qk_normalized=False), 66)
    s0 = initial_state(N, H, d, d, 6)
    say("case recurrent repeated", "N", N, "T", T, "H", H, "d", d)
    o1, st1 = run_rec(x, s0, l2=True)
    o2, st2 = run_rec(x, s0, l2=True)
    assert np.array_equal(o1, o2) and np.array_equal(st1, st2)


def test_prefill_then_decode():
    # the chunked forward leaves the final state; decoding continues from it
    H, d, T0, T1 = 2, 128, 200, 3
    x = gi.make_inputs(small_cfg("bf16", d, B=1, T=T0 + T1, H=H), 64)
    pre = dict(x, q=x["q"][:, :T0], k=x["k"][:, :T0], v=x["v"][:, :T0], g=x["g"][:, :T0], beta=x["beta"][:, :T0])
    dec = dict(x, q=x["q"][:, T0:], k=x["k"][:, T0:], v=x["v"][:, T0:], g=x["g"][:, T0:], beta=x["beta"][:, T0:])
    dp = dev_inputs(pre)
    _, ht = gdn.fwd(dp["q"], dp["k"], dp["v"], dp["g"], dp["beta"])
    o, st = run_rec(dec, to_np(ht))
    ro, rht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"])
    say("case recurrent after a chunked prefill of", T0)
    check_pair("o", o, ro[:, T0:], "bf16", "maxrel")
    check_pair("state", st, rht, "bf16", "frob")


def test_long_single_call():
    x = gi.make_inputs(small_cfg("fp32", 64, dv=128, B=2, T=300, H=2), 65)
    s0 = initial_state(2, 2, 64, 128, 5, std=0.1)
    o, st = run_rec(x, s0, l2=False)
    ro, rht = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0)
    check_pair("o", o, ro, "fp32", "maxrel")
    check_pair("state", st, rht, "fp32", "frob")


def test_decode_workload_sampled_sequences():
    # the decoding workload of the benchmark, in its launch configuration:
    # 256 sequences x 1 token, H = 16, d = 128, bf16, fp32 states in place;
    # sampled sequences (every head) against the oracle
    N, H, d = 256, 16, 128
    x = gi.make_inputs(gi.Config("decode", N, 1, H, d, d, "bf16", h0_std=0.1), 0)
    say("case recurrent decode workload N", N, "H", H, "d", d)
    o, st = run_rec(x, x["h0"])
    pick = [0, 1, 63, 64, 127, 128, 200, 255]
    ro, rht = oracle.fwd(x["q"][pick], x["k"][pick], x["v"][pick], x["g"][pick], x["beta"][pick], x["h0"][pick])
    check_pair("o", o[pick], ro, "bf16", "maxrel")
    check_pair("state", st[pick], rht, "bf16", "frob")
