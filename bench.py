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
ORACLE_THREADS = 16            # the host's CPU share for one GPU
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
C = 64


def kernel_bytes(D, E, units, state_units, with_ht=True):
    """Bytes each kernel reads and writes per launch, counting every tensor it
    touches once at storage size, the forward/backward context records in the
    workspace included (the kernels' own data-movement model).  Per (chunk,
    head) unit unless noted; state kernels add their per-(sequence, head) state
    I/O."""
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


def op_bytes(D, E, units, state_units, with_ht=True):
    """The operator's algorithmic bytes (its inputs read once and its outputs
    written once, nothing of the workspace), per launch of the kernel that
    moves them.  Per token and head: the forward reads q, k, v (3DE) and g,
    beta and writes o (DE): 1,032 B at D = 128 in bf16; the backward reads q,
    k, v, dO (4DE) and g, beta and writes dq, dk, dv (3DE) and dg, dbeta:
    1,808 B.  The backward's bytes all go through bwd_grad (which reads g as
    the chunk decays); of the forward's, fwd_prep reads k, v, g, beta and
    fwd_out reads q, k and writes o (k is an input of both); the state passes
    move only the states."""
    per_tok = {
        "fwd_prep": 2 * D * E + 8,
        "fwd_out": 3 * D * E,
        "bwd_prep": 0,
        "bwd_grad": 7 * D * E + 16,
        "fwd_state": 0,
        "bwd_state": 0,
    }
    per_unit = {k: v * C for k, v in per_tok.items()}
    out = {k: v * units for k, v in per_unit.items()}
    if with_ht:
        out["fwd_state"] += state_units * D * D * 4
    return out, per_unit


def kernel_flops(D, units):
    """Algorithmic flops per launch (2mnk per product, triangular operands at
    one half, no recompute, no transposes), split by kernel so that the six
    sum to the operator's 5C^2 D + 6C D^2 + C^3/3 (forward) and 12C^2 D +
    12C D^2 + 2C^3/3 (backward) per chunk: 438,272 per token and head at
    C = 64, D = 128."""
    per_unit = {
        # K K^T (lower), the solve, W = T Xw, U = T Xu
        "fwd_prep": C * C * D + C ** 3 // 3 + 2 * C * C * D,
        # W h, Kt^T V'
        "fwd_state": 4 * C * D * D,
        # Q h, Q K^T (lower), P V'
        "fwd_out": 2 * C * D * D + 2 * C * C * D,
        # P = Q K^T recomputed (lower), P^T dO, Z = (Gam Q)^T dO
        "bwd_prep": 2 * C * C * D + 2 * C * D * D,
        # Kt H', W^T dV'
        "bwd_state": 4 * C * D * D,
        # dP, dQ, dK, dW, dT, T^T dW, T^T dU, dA, K K^T and (E + E^T) K
        "bwd_grad": 10 * C * C * D + 6 * C * D * D + 2 * C ** 3 // 3,
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
    nthreads = min(ORACLE_THREADS, os.cpu_count() or 1)
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
    out = {"value": reps * tokens / el, "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": "%d complete fwd+bwd passes of the B=1,T=4096,H=16,d=128 workload%s%s "
                     "(fp64 token recurrence; %.1f s wall)"
                     % (reps, " with the conv1d" if cv is not None else "",
                        " with the gated RMSNorm" if gn is not None else "", el)}
    out.update(cpu_info())
    out["threads_note"] = "threads = min(%d, N*H): the host's CPU share for one GPU" % ORACLE_THREADS
    return out


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


def measured_peaks(torch, dev, reps=5):
    """Peaks of this GPU measured by the microbenchmarks of libgdn_peak.so (dense bf16
    MFMA issue on independent accumulators; a 2 GiB streaming copy and read, 16 bytes
    per lane), each the median of `reps` runs timed with events on the current stream.
    Also one wave's LDS reads and MFMAs in shader-clock cycles (medians of `reps` runs):
    per 1 KiB ds_read_b128 alone, per such read with one v_mfma_f32_16x16x32_bf16 after it
    (order pinned), and per MFMA alone (four independent accumulator chains).
    Returns {"mfma_bf16_TFLOPs", "hbm_copy_GBps", "hbm_read_GBps",
    "lds_read_cycles_one_wave", "lds_read_mfma_cycles_one_wave", "mfma_cycles_one_wave"}."""
    import numpy as np
    path = os.path.join(ROOT, "linear_attention_gated_amd", "libgdn_peak.so")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.gdn_peak_mfma_bf16.argtypes = [P, ctypes.c_int, ctypes.c_int, P]
    lib.gdn_peak_copy.argtypes = [P, P, ctypes.c_size_t, ctypes.c_int, P]
    lib.gdn_peak_read.argtypes = [P, ctypes.c_size_t, P, ctypes.c_int, P]
    lib.gdn_peak_lds_wave.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = P(torch.cuda.current_stream(dev).cuda_stream)

    def med(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return float(np.median(ts))

    def ok(rc):
        if rc != 0:
            raise RuntimeError("peak microbenchmark launch failed (hipError %d)" % rc)

    blocks, iters = 4 * cus, 2000       # four 4-wave workgroups per CU: four waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    t = med(lambda: ok(lib.gdn_peak_mfma_bf16(P(out.data_ptr()), blocks, iters, stream)))
    mfma = blocks * 4 * iters * 8 * 16384 / t / 1e12
    nbytes = 2 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a.fill_(1)
    sink = torch.empty(8 * cus * 256, dtype=torch.int32, device=dev)
    tc = med(lambda: ok(lib.gdn_peak_copy(P(a.data_ptr()), P(b.data_ptr()), nbytes, 8 * cus, stream)))
    tr = med(lambda: ok(lib.gdn_peak_read(P(a.data_ptr()), nbytes, P(sink.data_ptr()), 8 * cus, stream)))
    del a, b, sink, out
    cyc = torch.zeros(1, dtype=torch.int64, device=dev)
    lsink = torch.zeros(64, dtype=torch.int32, device=dev)
    lds = []
    for mode in (0, 1, 2):
        per = []
        for _ in range(reps):
            ok(lib.gdn_peak_lds_wave(P(cyc.data_ptr()), P(lsink.data_ptr()), mode, 256, stream))
            torch.cuda.synchronize()
            per.append(int(cyc.item()) / (256 * 32))
        lds.append(round(float(np.median(per)), 1))
    return {"mfma_bf16_TFLOPs": round(mfma, 1), "hbm_copy_GBps": round(2 * nbytes / tc / 1e9, 1),
            "hbm_read_GBps": round(nbytes / tr / 1e9, 1), "lds_read_cycles_one_wave": lds[0],
            "lds_read_mfma_cycles_one_wave": lds[1], "mfma_cycles_one_wave": lds[2]}


def cpu_info():
    """CPU model and counts of the host (the oracle's baseline runs on it)."""
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": aff}


def graph_step(torch, step, steps, warmup, tokens):
    """The step captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed `steps`
    times: {"ms_per_step", "tokens_per_s"}, or {"error"} if the capture fails (an optional
    figure that must not cost the bench line)."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step()
        for _ in range(warmup):
            gr.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            gr.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        return {"ms_per_step": round(1e3 * el / steps, 4), "tokens_per_s": round(tokens * steps / el, 1)}
    except RuntimeError as e:
        torch.cuda.synchronize()
        return {"error": str(e)[:200]}


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
        pk = measured_peaks(torch, dev)
        best = max(pk["hbm_copy_GBps"], pk["hbm_read_GBps"])
        roofline["measured_peak"] = best
        roofline["frac_of_measured_peak"] = round(a_gbs / best, 4)
        roofline["measured_peaks"] = pk
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
        nthreads = min(ORACLE_THREADS, os.cpu_count() or 1)
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
        cpu.update(cpu_info())
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


def config_sweep(args):
    """Every workload configuration once: the GPU path's time per call (median of 20, warm:
    calls back to back; cold: 1 GiB written before each call, outside the events), its
    error against the fp64 oracle, and the oracle's own time on the host (median of 3 on
    the CPU share of one GPU, plus one single-thread run of the T=4096 forward).  Prints
    one JSON line; not the headline."""
    import numpy as np
    import torch

    import gdn_inputs as gi
    import linear_attention_gated_amd as gdn
    import oracle

    dev = torch.device("cuda:0")
    nthreads = min(ORACLE_THREADS, os.cpu_count() or 1)

    def t(a, dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(dev)

    def err(a, ref, kind):
        a = a.detach().double().cpu().numpy()
        if kind == "frob":
            return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))
        return float(np.max(np.abs(a - ref)) / np.max(np.abs(ref)))

    def med_wall(fn, n=3):
        ts = []
        for _ in range(n):
            t0 = time.perf_counter()
            r = fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)), r

    rows = {}
    for name in ("c0", "c1", "c2", "c3", "c4"):
        cfg = gi.CONFIGS[name]
        x = gi.make_inputs(cfg, 0)
        dt = torch.float32 if cfg.dtype == "fp32" else torch.bfloat16
        q, k, v = (t(x[n_], dt) for n_ in ("q", "k", "v"))
        g, beta, h0 = t(x["g"], torch.float32), t(x["beta"], torch.float32), t(x["h0"], torch.float32)
        cu = None if x["cu_seqlens"] is None else (torch.from_numpy(x["cu_seqlens"]), t(x["cu_seqlens"], torch.int32))
        tokens = x["B"] * x["T"]
        p = gdn.make_problem(q, v, cu_host=None if cu is None else cu[0], cu_dev=None if cu is None else cu[1])
        wsf = torch.empty(gdn.lib().gdn_fwd_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8, device=dev)
        if cfg.with_grad:
            do = t(x["do"], dt)
            wsb = torch.empty(gdn.lib().gdn_bwd_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8, device=dev)

            def call():
                o, ht, ctx = gdn.fwd(q, k, v, g, beta, initial_state=h0, cu_seqlens=cu, return_context=True,
                                     workspace=wsf)
                return (o, ht) + tuple(gdn.bwd(q, k, v, g, beta, do, initial_state=h0, cu_seqlens=cu,
                                               context=ctx, workspace=wsb))
        else:
            def call():
                return gdn.fwd(q, k, v, g, beta, initial_state=h0, cu_seqlens=cu, workspace=wsf)
        got = call()
        torch.cuda.synchronize()
        warm = step_percentiles(torch, dev, call, 20, 0)
        cold = step_percentiles(torch, dev, call, 20, 1 << 30)
        ot, ref = med_wall(lambda: oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"],
                                              cu_seqlens=x["cu_seqlens"], nthreads=nthreads))
        errs = {"o_maxrel": err(got[0], ref[0], "maxrel")}
        errs["ht_maxrel" if cfg.dtype == "fp32" else "ht_frob"] = err(got[1], ref[1], "maxrel" if cfg.dtype == "fp32" else "frob")
        if cfg.with_grad:
            bt, rg = med_wall(lambda: oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], x["h0"],
                                                 cu_seqlens=x["cu_seqlens"], nthreads=nthreads))
            ot += bt
            for n_, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got[2:], rg):
                errs[n_ + "_maxrel"] = err(a, b, "maxrel")
                errs[n_ + "_frob"] = err(a, b, "frob")
        row = {"pass": "fwd+bwd" if cfg.with_grad else "fwd", "tokens": tokens, "H": x["H"], "d": x["dk"],
               "dtype": cfg.dtype, "sequences": x["N"],
               "gpu_warm_ms": warm["median_ms"], "gpu_cold_ms": cold["median_ms"],
               "gpu_warm_tokens_per_s": round(tokens / (warm["median_ms"] * 1e-3), 1),
               "gpu_cold_tokens_per_s": round(tokens / (cold["median_ms"] * 1e-3), 1),
               "oracle_s": round(ot, 3), "oracle_tokens_per_s": round(tokens / ot, 1),
               "oracle_threads": oracle.threads_used(x["N"], x["H"], nthreads),
               "errors": {k_: float("%.3e" % v_) for k_, v_ in errs.items()}}
        if name == "c1":
            st, _ = med_wall(lambda: oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], nthreads=1), n=1)
            row["oracle_single_thread_s"] = round(st, 3)
            row["oracle_single_thread_tokens_per_s"] = round(tokens / st, 1)
        rows[cfg.name] = row
        print("config %s: %s" % (cfg.name, json.dumps(row)), file=sys.stderr, flush=True)
        del x, q, k, v, got, ref
    out = {"metric": "per-configuration GPU time, parity and oracle time", "unit": "tokens/s", "n_gpus": 1,
           "higher_is_better": True, "data": "synthetic", "configs": rows, "host": cpu_info(),
           "oracle_threads_max": nthreads, "sources_sha": sources_sha()}
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
    ap.add_argument("--configs", action="store_true",
                    help="instead: every workload configuration once (GPU time warm and cold, error "
                         "against the oracle, the oracle's own time); not the headline")
    ap.add_argument("--no-profile-pass", action="store_true",
                    help="skip the second, event-bracketed timing region")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: runs on one GPU only (the operator's sequences and heads "
              "would shard across GPUs without any exchange, but no multi-GPU path is built); "
              "got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.decode:
        return decode_bench(args)
    if args.configs:
        return config_sweep(args)

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
        obytes, per_unit_o = op_bytes(D, 2, units, B * H)
        kflops = kernel_flops(D, units)
        for name in tot:
            avg_us = 1e3 * tot[name] / num[name]
            kernels[name] = {"avg_us": round(avg_us, 2), "launches_per_step": num[name] / args.steps}
            if obytes.get(name):
                kernels[name]["op_GBps"] = round(obytes[name] / (avg_us * 1e-6) / 1e9, 1)
            if name in kbytes:
                kernels[name]["moved_GBps"] = round(kbytes[name] / (avg_us * 1e-6) / 1e9, 1)
            if name in kflops:
                kernels[name]["achieved_TFLOPs"] = round(kflops[name] / (avg_us * 1e-6) / 1e12, 2)
        # the dominant kernel (longest), against the HBM roofline by the operator's own bytes
        dom = max((k_ for k_ in tot if obytes.get(k_)), key=lambda k_: tot[k_])
        avg_s = 1e-3 * tot[dom] / num[dom]
        a_gbs = obytes[dom] / avg_s / 1e9
        tr = traffic_for(dom)
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(a_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(a_gbs / HBM_PEAK_GBS, 4),
                    "traffic": tr, "algorithmic_bytes_per_launch": obytes[dom],
                    "units_per_launch": units, "bytes_per_unit": per_unit_o[dom],
                    "bytes_per_token_head": per_unit_o[dom] // C, "avg_us": round(avg_s * 1e6, 2),
                    "traffic_over_algorithmic": None if tr is None else round(tr / obytes[dom], 3),
                    # every tensor the kernel moves, its workspace records included
                    "moved_model": {"bytes_per_unit": per_unit_b[dom], "bytes_per_launch": kbytes[dom],
                                    "GBps": round(kbytes[dom] / avg_s / 1e9, 1),
                                    "frac": round(kbytes[dom] / avg_s / 1e9 / HBM_PEAK_GBS, 4)}}
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
        for tm in timing.values():
            tm["tokens_per_s_at_median"] = round(B * T / (tm["median_ms"] * 1e-3), 1)
        pk = measured_peaks(torch, dev)
        best = max(pk["hbm_copy_GBps"], pk["hbm_read_GBps"])
        if roofline is not None:
            roofline["measured_peak"] = best
            roofline["frac_of_measured_peak"] = round(roofline["achieved"] / best, 4)
            roofline["measured_peaks"] = pk
        if step_roof is not None:
            step_roof["mfma_frac_of_measured_peak"] = round(
                step_roof["achieved_TFLOPs"] / pk["mfma_bf16_TFLOPs"], 5)

    # the same step with gdn_bwd recomputing the forward context (no saved context), as the
    # backward runs when the forward's workspace is not kept
    recompute = None
    if not args.no_profile_pass and cv is None and gn is None:
        def step_rc():
            gdn.fwd(q, k, v, g, beta, workspace=wsf, qk_l2norm=l2)
            return gdn.bwd(q, k, v, g, beta, do, need_dh0=False, workspace=wsb, qk_l2norm=l2)
        for _ in range(args.warmup):
            step_rc()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            step_rc()
        torch.cuda.synchronize()
        el_rc = time.perf_counter() - t1
        recompute = {"ms_per_step": round(1e3 * el_rc / args.steps, 4),
                     "tokens_per_s": round(B * T * args.steps / el_rc, 1)}

    # the same step captured once in a HIP graph and replayed: the kernels without the host's
    # per-launch work (the headline value stays the eager step)
    graph = None if args.no_profile_pass else graph_step(torch, step, args.steps, args.warmup, B * T)

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
        "step_timing": timing, "recompute_step": recompute, "graph_step": graph,
        "sources_sha": sources_sha(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
