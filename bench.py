#!/usr/bin/env python3
"""GDN forward+backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = gdn_fwd (with the final state, keeping its forward context) then
gdn_bwd (reusing that context, no dh0) on the B=1, T=4096, H=16, d_k=d_v=128
bf16 workload with synthetic seeded inputs resident in HBM.  W untimed steps,
then K steps timed between two device synchronisations; value = tokens / s.
A second timed region of K steps brackets every kernel with HIP events on
the launch stream (through the library's gdn_profile_events hook) for the
per-kernel averages and the roofline of the dominant kernel.  The fp64 CPU
oracle is timed on the host beside it.  Prints one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN fwd+bwd tokens/s at T=4096,H=16,d=128 bf16; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
C = 64


def kernel_bytes(D, E, units, state_units, with_ht=True):
    """Algorithmic HBM bytes per launch of each kernel: each input it needs
    read once and each output written once, at storage size.  Per
    (chunk, head) unit unless noted; state kernels add their per-(sequence,
    head) state I/O."""
    per_unit = {
        # reads K, V (2CD E), g, beta; writes gamma, -W, Kt^T, U (3CD E), T (C^2 fp32)
        "fwd_prep": 5 * C * D * E + 3 * C * 4 + C * C * 4,
        # reads -W, Kt^T, U (3CD E), gamma_L; writes h (D^2 E), V' (CD E)
        "fwd_state": 4 * C * D * E + D * D * E + 4,
        # reads Q, K, V' (3CD E), h (D^2 E), gamma; writes O (CD E)
        "fwd_out": 4 * C * D * E + D * D * E + C * 4,
        # reads Q, K, dO, -W (4CD E), gamma; writes Kt, -W^T (2CD E), Z (D^2 E), dV'loc (CD E)
        "bwd_prep": 7 * C * D * E + D * D * E + C * 4,
        # reads Kt, -W^T (2CD E), Z (D^2 E), dV'loc (CD E), gamma; writes H' (D^2 E), dV' (CD E)
        "bwd_state": 4 * C * D * E + 2 * D * D * E + C * 4,
        # reads Q, K, V, dO, V', dV' (6CD E), h, H' (2 D^2 E), T (C^2 fp32), gamma, beta;
        # writes dQ, dK, dV (3CD E), dg, dbeta
        "bwd_grad": 9 * C * D * E + 2 * D * D * E + C * C * 4 + 4 * C * 4,
        # gated RMSNorm on the output, per C rows: reads x, z; writes y
        "gnorm_fwd": 3 * C * D * E,
        # reads x, z, dy; writes dx, dz (the dw partials are per workgroup, not counted)
        "gnorm_bwd": 5 * C * D * E,
        # causal conv1d on q, k, v side by side (three heads' D channels per unit): reads x, writes y
        "conv_fwd": 3 * 2 * C * D * E,
        # reads x, dy; writes dx (the dw/dbias partials are per workgroup, not counted)
        "conv_bwd": 3 * 3 * C * D * E,
    }
    out = {k: v * units for k, v in per_unit.items()}
    if with_ht:
        out["fwd_state"] += state_units * D * D * 4
    return out, per_unit


def kernel_flops(D, units):
    """Algorithmic flops per launch (2mnk per product, triangular operands at
    one half, no recompute, no transposes)."""
    per_unit = {
        "fwd_prep": C * C * D + C ** 3 // 3 + 2 * C * C * D,
        "fwd_state": 4 * C * D * D,
        "fwd_out": 2 * C * D * D + 2 * C * C * D,
        "bwd_prep": 2 * C * C * D + 2 * C * D * D,
        "bwd_state": 4 * C * D * D,
        "bwd_grad": 8 * C * D * D + 8 * C * C * D + 2 * C ** 3 // 3,
    }
    return {k: v * units for k, v in per_unit.items()}


def sources_sha():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "linear_attention_gated_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, summary="hbm_traffic_fwdbwd_T4096_H16_d128_bf16.txt"):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE from rocprofv3
    counter runs, scaled by a plain device copy of known size), read from the
    committed summary of the workload; None if there is none or the kernel
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", summary)
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    sha = None
    found = None
    for ln in lines:
        f = ln.split()
        if len(f) == 2 and f[0] == "sources_sha":
            sha = f[1]
        if len(f) == 6 and f[0] == "traffic" and f[1] == kernel:
            found = float(f[3]) + float(f[5])
    if sha != sources_sha() or found is None:
        return None
    return round(found)


def cpu_baseline(x, budget_s=10.0, max_reps=20, l2=False, gn=None, cv=None):
    import numpy as np

    import oracle
    nthreads = min(16, os.cpu_count() or 1)
    used = oracle.threads_used(x["N"], x["H"], nthreads)
    reps = 0
    t0 = time.perf_counter()
    while True:
        qkv = [x["q"], x["k"], x["v"]]
        if cv is not None:
            y = oracle.causal_conv1d_fwd(cv["x"], cv["w"])
            w_ = x["q"].shape[2] * x["q"].shape[3]
            qkv = [y[..., i * w_:(i + 1) * w_].reshape(x["q"].shape) for i in range(3)]
        o, _ = oracle.fwd(*qkv, x["g"], x["beta"], nthreads=nthreads, qk_l2norm=l2)
        do = x["do"]
        if gn is not None:
            oracle.gated_rmsnorm_fwd(o, gn["z"].reshape(o.shape), gn["w"])
            do = oracle.gated_rmsnorm_bwd(o, gn["z"].reshape(o.shape), gn["w"], gn["dy"].reshape(o.shape))[0]
        grads = oracle.bwd(*qkv, x["g"], x["beta"], do, nthreads=nthreads, qk_l2norm=l2)
        if cv is not None:
            dqkv = np.concatenate([gq.reshape(cv["x"].shape[:2] + (-1,)) for gq in grads[:3]], axis=-1)
            oracle.causal_conv1d_bwd(cv["x"], cv["w"], dqkv)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            break
    tokens = x["B"] * x["T"]
    return {"value": reps * tokens / el, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": "%d complete fwd+bwd passes of the B=1,T=4096,H=16,d=128 workload%s%s "
                      "(fp64 token recurrence; %.1f s wall)"
                      % (reps, " with the conv1d" if cv is not None else "",
                         " with the gated RMSNorm" if gn is not None else "", el)}


class HipEvents:
    """A few hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev[i] = h
        self.n = n

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.ev[i])


def copy_calibration(torch, dev, nbytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling HBM byte counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a.fill_(1)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copy calibration: %d x %d bytes" % (reps, nbytes), file=sys.stderr)


def measured_peak_gbs(torch, dev, nbytes=1 << 30, reps=5):
    """HBM bandwidth that library kernels reach on this GPU, the measured peak beside the
    vendor one: a 1 GiB device-to-device copy (bytes read plus written) and a 1 GiB fp32
    sum (bytes read), each the median of `reps`.  Returns (best, copy, read) in GB/s."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a.fill_(1)
    af = a.view(torch.float32)

    def med(fn, moved):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return moved / sorted(ts)[reps // 2] / 1e9

    cp = med(lambda: b.copy_(a), 2 * nbytes)
    rd = med(lambda: af.sum(), nbytes)
    del a, b, af
    return max(cp, rd), cp, rd


def step_percentiles(torch, dev, step, n, flush_bytes):
    """Per-step times (ms) over n steps, each bracketed by events on the current stream;
    with flush_bytes > 0 a write of that many bytes runs before each step, outside the
    events, so that the step starts with nothing of its own in the L2 and memory-side caches."""
    import numpy as np
    junk = torch.empty(flush_bytes, dtype=torch.uint8, device=dev) if flush_bytes else None
    ts = []
    for _ in range(n):
        if junk is not None:
            junk.fill_(0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del junk
    q = np.percentile(np.array(ts), [10, 50, 90])
    return {"steps": n, "p10_ms": round(float(q[0]), 4), "median_ms": round(float(q[1]), 4),
            "p90_ms": round(float(q[2]), 4)}


def decode_bench(args):
    """One step = one recurrent call: N sequences x 1 new token, H=16, d_k=d_v=128, bf16, the
    fp32 states [N,16,128,128] read and written in place."""
    import numpy as np
    import torch

    import gdn_inputs as gi
    import linear_attention_gated_amd as gdn

    N, H, D = args.decode, 16, 128
    cfg = gi.Config("decode", N, 1, H, D, D, "bf16", h0_std=0.1)
    x = gi.make_inputs(cfg, 0)
    dev = torch.device("cuda:0")

    def t(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    q, k, v = (t(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    g, beta = t(x["g"], torch.float32), t(x["beta"], torch.float32)
    state = t(x["h0"], torch.float32)
    L = gdn.lib()
    for _ in range(args.warmup):
        gdn.recurrent_fwd(q, k, v, g, beta, state)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gdn.recurrent_fwd(q, k, v, g, beta, state)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_per_step = 1e3 * el / args.steps
    # algorithmic bytes: the state both ways, q, k, v read and o written, g and beta
    byts = N * H * (2 * D * D * 4 + 4 * D * 2 + 8)
    roofline = None
    if not args.no_profile_pass:
        evs = HipEvents(2 * args.steps)
        L.gdn_profile_events(ctypes.cast(evs.ev, ctypes.c_void_p), args.steps)
        for _ in range(args.steps):
            gdn.recurrent_fwd(q, k, v, g, beta, state)
        torch.cuda.synchronize()
        cnt = L.gdn_profile_count()
        L.gdn_profile_events(None, 0)
        avg_us = 1e3 * sum(evs.elapsed_ms(2 * i, 2 * i + 1) for i in range(cnt)) / cnt
        evs.close()
        a_gbs = byts / (avg_us * 1e-6) / 1e9
        roofline = {"kernel": "recurrent", "bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(a_gbs / HBM_PEAK_GBS, 4),
                    "traffic": traffic_for("recurrent", "hbm_traffic_decode_N%d_T1_H16_d128_bf16.txt" % N),
                    "algorithmic_bytes_per_launch": byts, "units_per_launch": N * H,
                    "bytes_per_unit": byts // (N * H), "avg_us": round(avg_us, 2)}
        best, cp, rd = measured_peak_gbs(torch, dev)
        roofline["measured_peak"] = round(best, 1)
        roofline["frac_of_measured_peak"] = round(a_gbs / best, 4)
        roofline["measured_copy_GBps"] = round(cp, 1)
        roofline["measured_read_GBps"] = round(rd, 1)
        # back to back, part of the state pool is still in the memory-side cache
        # from the previous call; "cold" writes 1 GiB before each call (as the
        # rest of a model would between two decoding steps)
        call = lambda: gdn.recurrent_fwd(q, k, v, g, beta, state)
        timing = {"warm": step_percentiles(torch, dev, call, 30, 0),
                  "cold": step_percentiles(torch, dev, call, 30, 1 << 30)}
        for tm in timing.values():
            tm["GBps_at_median"] = round(byts / (tm["median_ms"] * 1e-3) / 1e9, 1)
    if args.copy_calib:
        copy_calibration(torch, dev)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = min(16, os.cpu_count() or 1)
        reps, c0 = 0, time.perf_counter()
        while True:
            oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], nthreads=nthreads)
            reps += 1
            ce = time.perf_counter() - c0
            if ce >= 5.0 or reps >= 50:
                break
        cpu = {"value": reps * N / ce, "unit": "tokens/s", "cores": oracle.threads_used(N, H, nthreads),
               "kind": "oracle", "sample": "%d complete decode steps of the same workload (fp64 token "
               "recurrence; %.1f s wall)" % (reps, ce)}
    out = {
        "metric": "GDN recurrent decode tokens/s", "value": round(N * args.steps / el, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gdn_decode_N%d_T1_H16_d128_bf16_state_inplace" % N, "N": N, "H": H, "dk": D,
                   "dv": D, "parallelism": "none (1 GPU)"},
        "roofline": roofline, "cpu_baseline": cpu, "sources_sha": sources_sha(),
    }
    if roofline is not None:
        out["step_timing"] = timing
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--qk-l2norm", action="store_true",
                    help="raw q/k rows, normalised inside the operator (not the headline workload)")
    ap.add_argument("--gated-norm", action="store_true",
                    help="the output gate's RMSNorm in the step (forward after the operator, its "
                         "backward feeding the operator's); not the headline workload")
    ap.add_argument("--conv", action="store_true",
                    help="the layer's causal conv1d (K=4, SiLU) on raw q, k, v projections before the "
                         "operator, its backward after; implies --qk-l2norm; not the headline workload")
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="instead: the recurrent (decoding) forward, N sequences of one new token "
                         "each with their states in place (H=16, d=128, bf16)")
    ap.add_argument("--no-profile-pass", action="store_true",
                    help="skip the second, event-bracketed timing region")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the operator's sequences and heads "
              "would shard across GPUs without any exchange, but no multi-GPU path is built); "
              "got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.decode:
        return decode_bench(args)

    import numpy as np
    import torch

    import gdn_inputs as gi
    import linear_attention_gated_amd as gdn

    dev = torch.device("cuda:0")
    cfg = gi.CONFIGS["metric"]
    l2 = bool(args.qk_l2norm or args.conv)
    if l2:
        import dataclasses
        cfg = dataclasses.replace(cfg, qk_normalized=False)
    x = gi.make_inputs(cfg, 0)
    B, T, H, D = x["B"], x["T"], x["H"], x["dk"]

    def t(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    q, k, v, do = (t(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    g, beta = t(x["g"], torch.float32), t(x["beta"], torch.float32)
    cv = None
    if args.conv:
        # raw projections of q, k, v side by side, [B, T, 3*H*D] channels last, and the conv
        # weights; one conv call covers all three, the operator reads slices of its output
        cv = gi.make_conv_inputs(B, T, 3 * H * D, 4, "bf16", seed=20)
        cvx = t(cv["x"], torch.bfloat16)
        cvw = t(cv["w"], torch.float32)
        pc = gdn.make_conv_problem(cvx, 4)
        wsc = torch.empty(gdn.lib().gdn_causal_conv1d_bwd_workspace_bytes(ctypes.byref(pc)), dtype=torch.uint8,
                          device=dev)
    gn = None
    if args.gated_norm:
        gn = gi.make_gated_norm_inputs(B * T * H, D, "bf16", seed=1, x=np.zeros((B * T * H, D)))
        zt = t(gn["z"].reshape(B, T, H, D), torch.bfloat16)
        wt = t(gn["w"], torch.float32)
        dyt = t(gn["dy"].reshape(B, T, H, D), torch.bfloat16)
        pn = gdn.make_gated_norm_problem(zt)
    p = gdn.make_problem(q, v, qk_l2norm=l2)
    L = gdn.lib()
    wsf = torch.empty(L.gdn_fwd_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8, device=dev)
    wsb = torch.empty(L.gdn_bwd_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8, device=dev)

    if gn is not None:
        wsn = torch.empty(L.gdn_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(pn)), dtype=torch.uint8,
                          device=dev)

    def step():
        qq, kk, vv = q, k, v
        if cv is not None:
            y = gdn.causal_conv1d_fwd(cvx, cvw)
            qq, kk, vv = (y[..., i * H * D:(i + 1) * H * D].view(B, T, H, D) for i in range(3))
        o, ht, ctx = gdn.fwd(qq, kk, vv, g, beta, return_context=True, workspace=wsf, qk_l2norm=l2)
        dO = do
        if gn is not None:
            gdn.gated_rmsnorm_fwd(o, zt, wt)
            dO = gdn.gated_rmsnorm_bwd(o, zt, wt, dyt, workspace=wsn)[0]
        grads = gdn.bwd(qq, kk, vv, g, beta, dO, context=ctx, need_dh0=False, workspace=wsb, qk_l2norm=l2)
        if cv is not None:
            # dq, dk, dv are slices of one [B, T, 3*H*D] buffer laid out like the conv output
            dqkv = grads[0].as_strided((B, T, 3 * H * D), (T * 3 * H * D, 3 * H * D, 1), grads[0].storage_offset())
            gdn.causal_conv1d_bwd(cvx, cvw, dqkv, workspace=wsc)
        return grads

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_per_step = 1e3 * el / args.steps
    value = B * T * args.steps / el

    kernels = {}
    roofline = None
    step_roof = None
    units = int(np.sum(np.ceil(np.full(B, T) / C))) * H
    if not args.no_profile_pass:
        launches_per_step = 8 + (3 if gn is not None else 0) + (3 if cv is not None else 0)
        n = launches_per_step * args.steps
        evs = HipEvents(2 * n)
        L.gdn_profile_events(ctypes.cast(evs.ev, ctypes.c_void_p), n)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        cnt = L.gdn_profile_count()
        L.gdn_profile_events(None, 0)
        print("profile pass: %d launches bracketed" % cnt, file=sys.stderr)
        if cnt == 0:
            raise RuntimeError("the event-bracketed pass recorded no kernel launches")
        tot = {}
        num = {}
        for i in range(min(cnt, n)):
            name = L.gdn_profile_name(i).decode()
            ms = evs.elapsed_ms(2 * i, 2 * i + 1)
            tot[name] = tot.get(name, 0.0) + ms
            num[name] = num.get(name, 0) + 1
        evs.close()
        kbytes, per_unit_b = kernel_bytes(D, 2, units, B * H)
        kflops = kernel_flops(D, units)
        for name in tot:
            avg_us = 1e3 * tot[name] / num[name]
            kernels[name] = {"avg_us": round(avg_us, 2), "launches_per_step": num[name] / args.steps}
            if name in kbytes:
                kernels[name]["achieved_GBps"] = round(kbytes[name] / (avg_us * 1e-6) / 1e9, 1)
            if name in kflops:
                kernels[name]["achieved_TFLOPs"] = round(kflops[name] / (avg_us * 1e-6) / 1e12, 2)
        dom = max((k_ for k_ in tot if k_ in kbytes), key=lambda k_: tot[k_])
        a_gbs = kbytes[dom] / (1e-3 * tot[dom] / num[dom]) / 1e9
        tr = traffic_for(dom)
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(a_gbs / HBM_PEAK_GBS, 4),
                    "traffic": tr, "algorithmic_bytes_per_launch": kbytes[dom],
                    "units_per_launch": units, "bytes_per_unit": per_unit_b[dom]}
        # whole step: the operator's own input/output bytes per token and head
        step_bytes = (1032 + 1808) * B * T * H + B * H * D * D * 4
        step_flops = (140629 + 297643) * B * T * H
        step_roof = {"bytes": step_bytes, "achieved_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                     "hbm_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "flops": step_flops,
                     "achieved_TFLOPs": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
                     "mfma_frac": round(step_flops / (ms_per_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 5),
                     "kernel_sum_us": round(sum(1e3 * tot[k_] / args.steps for k_ in tot), 1)}
        # the sequential passes are latency-bound: their critical path is the dependent
        # chunk steps of the longest sequence times the time of one step
        nsteps = int(np.ceil(T / C))
        step_roof["critical_path"] = {
            k_: {"dependent_steps": nsteps, "us_per_step": round(1e3 * tot[k_] / num[k_] / nsteps, 3)}
            for k_ in ("fwd_state", "bwd_state") if k_ in tot}

    # per-step percentiles, warm (steps back to back) and cold (1 GiB written before each step)
    timing = None
    if not args.no_profile_pass:
        timing = {"warm": step_percentiles(torch, dev, step, 30, 0),
                  "cold": step_percentiles(torch, dev, step, 30, 1 << 30)}
        best, cp, rd = measured_peak_gbs(torch, dev)
        if roofline is not None:
            roofline["measured_peak"] = round(best, 1)
            roofline["frac_of_measured_peak"] = round(roofline["achieved"] / best, 4)
            roofline["measured_copy_GBps"] = round(cp, 1)
            roofline["measured_read_GBps"] = round(rd, 1)

    if args.copy_calib:
        copy_calibration(torch, dev)

    cpu = None if args.no_cpu_baseline else cpu_baseline(x, l2=l2, gn=gn, cv=cv)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gdn_fwdbwd_B1_T4096_H16_d128_bf16_chunk64" + ("_qkl2norm" if l2 else "")
                   + ("_conv1d" if cv is not None else "") + ("_gatednorm" if gn is not None else ""),
                   "B": B, "T": T, "H": H,
                   "dk": D, "dv": D, "chunk": C, "parallelism": "none (1 GPU)"},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels, "step_roofline": step_roof,
        "step_timing": timing,
        "sources_sha": sources_sha(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
