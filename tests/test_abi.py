"""The C ABI on the host: the library loads without a GPU, exports what
include/gdn.h declares, and rejects every invalid argument before any HIP
call.  CPU only: every call below is invalid by construction (each case breaks
exactly one check), so no kernel is ever launched on the fake pointers."""
import ctypes
import os
import re

import pytest

import linear_attention_gated_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    lib = gdn.lib()
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_peak_library_exports_its_header():
    # the measured-peak microbenchmarks live in a library of their own
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "gdn_peak.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))
    assert names == ["gdn_peak_copy", "gdn_peak_lds_wave", "gdn_peak_mfma_bf16", "gdn_peak_read"], names
    lib = ctypes.CDLL(os.path.join(ROOT, "linear_attention_gated_amd", "libgdn_peak.so"))
    for n in names:
        assert hasattr(lib, n), n
    # invalid arguments are rejected before any launch
    lib.gdn_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    assert lib.gdn_peak_copy(None, None, 16, 1, None) != 0
    lib.gdn_peak_lds_wave.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.gdn_peak_lds_wave(None, None, 0, 1, None) != 0
    assert lib.gdn_peak_lds_wave(ctypes.c_void_p(16), ctypes.c_void_p(16), 3, 1, None) != 0


def test_abi_version_and_status_strings():
    assert gdn.lib().gdn_abi_version() == 7
    assert gdn.status_string(0) == "GDN_OK"
    assert gdn.status_string(3) == "GDN_ERR_WORKSPACE_TOO_SMALL"


def test_problem_struct_layout():
    # int64 x7, two pointers, float, enum(int), two int32 -> 88 bytes on x86-64
    assert ctypes.sizeof(gdn.GdnProblem) == 88
    # int64 x2, float, enum(int) -> 24 bytes
    assert ctypes.sizeof(gdn.GdnGatedNormProblem) == 24
    # int64 x5, two pointers, int32, enum(int) -> 64 bytes
    assert ctypes.sizeof(gdn.GdnConvProblem) == 64


FAKE = 0x7f0000000000  # never dereferenced: every call below fails validation


def base_problem(**kw):
    p = gdn.GdnProblem()
    p.batch, p.seqlen, p.heads, p.dk, p.dv, p.chunk = 1, 256, 2, 64, 64, 64
    p.num_seqs = 0
    p.cu_seqlens_host = None
    p.cu_seqlens_dev = None
    p.scale = 1.0
    p.dtype = gdn.GDN_BF16
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def fwd_ptrs(p, ws_bytes=None, **over):
    T = p.batch * p.seqlen
    qk = T * p.heads * max(p.dk, 1) * (2 if p.dtype == gdn.GDN_BF16 else 4)
    gb = T * p.heads * 4
    sb = max(p.num_seqs if p.cu_seqlens_host else p.batch, 1) * p.heads * 64 * 64 * 4
    base = FAKE
    ptrs = {}
    for name, size in (("q", qk), ("k", qk), ("v", qk), ("g", gb), ("beta", gb), ("h0", sb),
                       ("o", qk), ("ht", sb)):
        ptrs[name] = base
        base += (size + 4095) // 4096 * 4096 + 4096
    ptrs["ws"] = base
    ptrs.update(over)
    need = gdn.lib().gdn_fwd_workspace_bytes(ctypes.byref(p))
    ws_bytes = need if ws_bytes is None else ws_bytes
    return ptrs, ws_bytes


def call_fwd(p, ws_bytes=None, **over):
    ptrs, wsb = fwd_ptrs(p, ws_bytes, **over)
    P = ctypes.c_void_p
    st = gdn.lib().gdn_fwd(ctypes.byref(p), P(ptrs["q"]), P(ptrs["k"]), P(ptrs["v"]), P(ptrs["g"]),
                           P(ptrs["beta"]), P(ptrs["h0"]), P(ptrs["o"]), P(ptrs["ht"]),
                           P(ptrs["ws"]), wsb, None)
    return st, gdn.last_error_message()


def test_workspace_query_valid_and_invalid():
    L = gdn.lib()
    p = base_problem()
    f = L.gdn_fwd_workspace_bytes(ctypes.byref(p))
    b = L.gdn_bwd_workspace_bytes(ctypes.byref(p))
    assert f > 0 and b > f and f % 256 == 0
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(base_problem(dk=96, dv=96))) == 0
    assert L.gdn_fwd_workspace_bytes(None) == 0
    # in-operator normalisation keeps the reciprocal key norms (one fp32 per token and head) in the
    # forward context and the query norms in the backward's own region
    fn = L.gdn_fwd_workspace_bytes(ctypes.byref(base_problem(qk_l2norm=1)))
    bn = L.gdn_bwd_workspace_bytes(ctypes.byref(base_problem(qk_l2norm=1)))
    assert fn >= f + 256 * 2 * 4 and fn % 256 == 0
    assert bn >= b + 2 * 256 * 2 * 4 and bn % 256 == 0


CASES = [
    ("dv_96", dict(dv=96), {}, gdn.GDN_ERR_UNSUPPORTED, "head dims"),
    ("dim_96", dict(dk=96, dv=96), {}, gdn.GDN_ERR_UNSUPPORTED, "head dims"),
    ("chunk_32", dict(chunk=32), {}, gdn.GDN_ERR_UNSUPPORTED, "chunk"),
    ("dtype_7", dict(dtype=7), {}, gdn.GDN_ERR_UNSUPPORTED, "dtype"),
    ("heads_0", dict(heads=0), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "heads"),
    ("batch_0", dict(batch=0), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "batch"),
    ("seqlen_neg", dict(seqlen=-1), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "seqlen"),
    ("scale_nan", dict(scale=float("nan")), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "scale"),
    ("null_q", {}, dict(q=0), gdn.GDN_ERR_INVALID_ARGUMENT, "q is NULL"),
    ("null_beta", {}, dict(beta=0), gdn.GDN_ERR_INVALID_ARGUMENT, "beta is NULL"),
    ("null_ws", {}, dict(ws=0), gdn.GDN_ERR_INVALID_ARGUMENT, "workspace is NULL"),
    ("misaligned_k", {}, dict(k=FAKE + 8), gdn.GDN_ERR_INVALID_ARGUMENT, "aligned"),
    ("misaligned_ws", {}, dict(ws=FAKE + (1 << 36) + 16), gdn.GDN_ERR_INVALID_ARGUMENT,
     "256-byte"),
    ("o_aliases_q", {}, dict(o=FAKE), gdn.GDN_ERR_INVALID_ARGUMENT, "overlaps"),
    ("ht_aliases_h0", {}, dict(ht="h0"), gdn.GDN_ERR_INVALID_ARGUMENT, "overlaps"),
    ("l2norm_2", dict(qk_l2norm=2), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "qk_l2norm"),
    ("stride_small", dict(qkv_token_stride=64), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "qkv_token_stride"),
    ("stride_odd", dict(qkv_token_stride=3 * 2 * 64 + 4), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "multiple"),
    ("stride_neg", dict(qkv_token_stride=-8), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "qkv_token_stride"),
]


@pytest.mark.parametrize("name,pkw,pover,status,msg", CASES, ids=[c[0] for c in CASES])
def test_invalid_arguments(name, pkw, pover, status, msg):
    p = base_problem(**pkw)
    if pover.get("ht") == "h0":
        ptrs, _ = fwd_ptrs(p)
        pover = dict(ht=ptrs["h0"] + 64)
    st, m = call_fwd(p, **pover)
    assert st == status, (st, m)
    assert msg in m, m


def test_workspace_too_small():
    p = base_problem()
    need = gdn.lib().gdn_fwd_workspace_bytes(ctypes.byref(p))
    st, m = call_fwd(p, ws_bytes=need - 256)
    assert st == gdn.GDN_ERR_WORKSPACE_TOO_SMALL, m


def _varlen(cu, **kw):
    arr = (ctypes.c_int32 * len(cu))(*cu)
    p = base_problem(seqlen=cu[-1], num_seqs=len(cu) - 1,
                     cu_seqlens_host=ctypes.addressof(arr), cu_seqlens_dev=FAKE + (1 << 40), **kw)
    return p, arr


@pytest.mark.parametrize("cu,msg", [([1, 5, 9], "cu_seqlens[0]"), ([0, 9, 5], "decreases"),
                                    ([0, 4, 9], None)])
def test_varlen_validation(cu, msg):
    p, arr = _varlen(cu)
    if msg is None:
        # consistent cu_seqlens, but seqlen disagrees with cu[N]
        p.seqlen = 10
        msg = "seqlen"
    st, m = call_fwd(p)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and msg in m, m


def test_varlen_needs_batch_one_and_both_copies():
    p, arr = _varlen([0, 4, 9], batch=2)
    st, m = call_fwd(p)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "batch" in m
    p, arr = _varlen([0, 4, 9])
    p.cu_seqlens_dev = None
    st, m = call_fwd(p)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "both" in m


def test_bwd_rejects_missing_outputs():
    p = base_problem()
    P = ctypes.c_void_p
    args = [P(FAKE + i * (1 << 30)) for i in range(15)]
    args[11] = None  # dg (order: q k v g beta h0 do dht dq dk dv dg dbeta dh0 fwd_ws)
    st = gdn.lib().gdn_bwd(ctypes.byref(p), *args, P(FAKE + (1 << 36)),
                           gdn.lib().gdn_bwd_workspace_bytes(ctypes.byref(p)), None)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "dg is NULL" in gdn.last_error_message()


# ---- gated RMSNorm entry points ---------------------------------------------

def gnorm_problem(**kw):
    p = gdn.GdnGatedNormProblem()
    p.rows, p.dim, p.eps, p.dtype = 300, 128, 1e-6, gdn.GDN_BF16
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def call_gnorm_bwd(p, **over):
    L = gdn.lib()
    ptrs = dict(x=FAKE, z=FAKE + (1 << 30), w=FAKE + (2 << 30), dy=FAKE + (3 << 30), dx=FAKE + (4 << 30),
                dz=FAKE + (5 << 30), dw=FAKE + (6 << 30), ws=FAKE + (7 << 30))
    ptrs.update(over)
    need = L.gdn_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(p))
    nb = over.get("ws_bytes", need)
    P = ctypes.c_void_p
    st = L.gdn_gated_rmsnorm_bwd(ctypes.byref(p), *(P(ptrs[n]) if ptrs[n] else None for n in
                                                    ("x", "z", "w", "dy", "dx", "dz", "dw", "ws")),
                                 nb, None)
    return st, gdn.last_error_message()


GNORM_CASES = [
    ("dim_96", dict(dim=96), {}, gdn.GDN_ERR_UNSUPPORTED, "dim"),
    ("dtype_5", dict(dtype=5), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "dtype"),
    ("rows_neg", dict(rows=-1), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "rows"),
    ("eps_neg", dict(eps=-1e-6), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "eps"),
    ("eps_inf", dict(eps=float("inf")), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "eps"),
    ("null_w", {}, dict(w=0), gdn.GDN_ERR_INVALID_ARGUMENT, "w is NULL"),
    ("null_dw", {}, dict(dw=0), gdn.GDN_ERR_INVALID_ARGUMENT, "dw is NULL"),
    ("misaligned_dy", {}, dict(dy=FAKE + (3 << 30) + 4), gdn.GDN_ERR_INVALID_ARGUMENT, "aligned"),
    ("dx_aliases_x", {}, dict(dx=FAKE + 256), gdn.GDN_ERR_INVALID_ARGUMENT, "overlaps"),
    ("dz_aliases_dx", {}, dict(dz=FAKE + (4 << 30) + 512), gdn.GDN_ERR_INVALID_ARGUMENT, "overlap"),
    ("ws_misaligned", {}, dict(ws=FAKE + (7 << 30) + 16), gdn.GDN_ERR_INVALID_ARGUMENT, "256-byte"),
    ("ws_small", {}, dict(ws_bytes=256), gdn.GDN_ERR_WORKSPACE_TOO_SMALL, "workspace"),
]


@pytest.mark.parametrize("name,pkw,pover,status,msg", GNORM_CASES, ids=[c[0] for c in GNORM_CASES])
def test_gated_norm_invalid_arguments(name, pkw, pover, status, msg):
    st, m = call_gnorm_bwd(gnorm_problem(**pkw), **pover)
    assert st == status, (st, m)
    assert msg in m, m


def test_gated_norm_forward_validation():
    L = gdn.lib()
    P = ctypes.c_void_p
    p = gnorm_problem()
    st = L.gdn_gated_rmsnorm_fwd(ctypes.byref(p), P(FAKE), P(FAKE + (1 << 30)), None, P(FAKE + (2 << 30)), None)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "w is NULL" in gdn.last_error_message()
    st = L.gdn_gated_rmsnorm_fwd(ctypes.byref(p), P(FAKE), P(FAKE + (1 << 30)), P(FAKE + (3 << 30)),
                                 P(FAKE + 64), None)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "overlaps" in gdn.last_error_message()
    st = L.gdn_gated_rmsnorm_fwd(None, None, None, None, None, None)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT


def test_gated_norm_workspace_size():
    L = gdn.lib()
    # one fp32 partial row of dw per backward workgroup, at most 1024 of them
    big = L.gdn_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(gnorm_problem(rows=1 << 20)))
    assert big == 1024 * 128 * 4
    assert L.gdn_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(gnorm_problem(rows=0))) == 512
    assert L.gdn_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(gnorm_problem(dim=96))) == 0


# ---- causal conv1d entry points ---------------------------------------------

def conv_problem(**kw):
    p = gdn.GdnConvProblem()
    p.batch, p.seqlen, p.channels, p.kernel_size, p.num_seqs = 2, 100, 64, 4, 0
    p.cu_seqlens_host = p.cu_seqlens_dev = None
    p.activation, p.dtype = 1, gdn.GDN_BF16
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def call_conv_bwd(p, **over):
    L = gdn.lib()
    ptrs = dict(x=FAKE, w=FAKE + (1 << 30), b=FAKE + (2 << 30), dy=FAKE + (3 << 30), dx=FAKE + (4 << 30),
                dw=FAKE + (5 << 30), db=FAKE + (6 << 30), ws=FAKE + (7 << 30))
    ptrs.update(over)
    need = L.gdn_causal_conv1d_bwd_workspace_bytes(ctypes.byref(p))
    P = ctypes.c_void_p
    st = L.gdn_causal_conv1d_bwd(ctypes.byref(p), *(P(ptrs[n]) if ptrs[n] else None for n in
                                                    ("x", "w", "b", "dy", "dx", "dw", "db", "ws")),
                                 over.get("ws_bytes", need), None)
    return st, gdn.last_error_message()


CONV_CASES = [
    ("k5", dict(kernel_size=5), {}, gdn.GDN_ERR_UNSUPPORTED, "kernel_size"),
    ("k0", dict(kernel_size=0), {}, gdn.GDN_ERR_UNSUPPORTED, "kernel_size"),
    ("c6", dict(channels=6), {}, gdn.GDN_ERR_UNSUPPORTED, "channels"),
    ("act2", dict(activation=2), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "activation"),
    ("dtype9", dict(dtype=9), {}, gdn.GDN_ERR_UNSUPPORTED, "dtype"),
    ("seqlen_neg", dict(seqlen=-3), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "seqlen"),
    ("batch0", dict(batch=0), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "batch"),
    ("null_w", {}, dict(w=0), gdn.GDN_ERR_INVALID_ARGUMENT, "w is NULL"),
    ("null_dx", {}, dict(dx=0), gdn.GDN_ERR_INVALID_ARGUMENT, "dx is NULL"),
    ("misaligned_x", {}, dict(x=FAKE + 8), gdn.GDN_ERR_INVALID_ARGUMENT, "aligned"),
    ("dx_aliases_dy", {}, dict(dx=FAKE + (3 << 30) + 128), gdn.GDN_ERR_INVALID_ARGUMENT, "overlaps"),
    ("db_aliases_dw", {}, dict(db=FAKE + (5 << 30) + 16), gdn.GDN_ERR_INVALID_ARGUMENT, "overlap"),
    ("ws_small", {}, dict(ws_bytes=256), gdn.GDN_ERR_WORKSPACE_TOO_SMALL, "workspace"),
    ("ws_misaligned", {}, dict(ws=FAKE + (7 << 30) + 64), gdn.GDN_ERR_INVALID_ARGUMENT, "256-byte"),
]


@pytest.mark.parametrize("name,pkw,pover,status,msg", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_conv_invalid_arguments(name, pkw, pover, status, msg):
    st, m = call_conv_bwd(conv_problem(**pkw), **pover)
    assert st == status, (st, m)
    assert msg in m, m


def test_conv_varlen_validation_and_workspace():
    arr = (ctypes.c_int32 * 4)(0, 30, 20, 100)
    p = conv_problem(batch=1, num_seqs=3, cu_seqlens_host=ctypes.addressof(arr), cu_seqlens_dev=FAKE + (1 << 40))
    st, m = call_conv_bwd(p)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "decreases" in m
    arr2 = (ctypes.c_int32 * 3)(0, 30, 100)
    p = conv_problem(batch=2, num_seqs=2, cu_seqlens_host=ctypes.addressof(arr2), cu_seqlens_dev=FAKE + (1 << 40))
    st, m = call_conv_bwd(p)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "batch" in m
    L = gdn.lib()
    # one fp32 partial per (grid row, channel, tap or bias), at most 64 grid rows
    big = L.gdn_causal_conv1d_bwd_workspace_bytes(ctypes.byref(conv_problem(batch=1, seqlen=1 << 20, channels=6144)))
    assert big == 64 * 6144 * 5 * 4
    assert L.gdn_causal_conv1d_bwd_workspace_bytes(ctypes.byref(conv_problem(kernel_size=7))) == 0


# ---- recurrent (decoding) entry point ------------------------------------------

def call_rec(p, num_slots=4, **over):
    ptrs = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), g=FAKE + (3 << 30), b=FAKE + (4 << 30),
                st=FAKE + (5 << 30), idx=None, o=FAKE + (7 << 30))
    ptrs.update(over)
    P = ctypes.c_void_p
    st = gdn.lib().gdn_recurrent_fwd(ctypes.byref(p), *(P(ptrs[n]) if ptrs[n] else None for n in
                                                     ("q", "k", "v", "g", "b", "st", "idx")),
                                     num_slots, P(ptrs["o"]) if ptrs["o"] else None, None)
    return st, gdn.last_error_message()


REC_CASES = [
    ("dk96", dict(dk=96, dv=96), {}, gdn.GDN_ERR_UNSUPPORTED, "dk"),
    ("dv256", dict(dv=256), {}, gdn.GDN_ERR_UNSUPPORTED, "dv"),
    ("l2norm3", dict(qk_l2norm=3), {}, gdn.GDN_ERR_INVALID_ARGUMENT, "qk_l2norm"),
    ("null_state", {}, dict(st=0), gdn.GDN_ERR_INVALID_ARGUMENT, "state is NULL"),
    ("o_aliases_v", {}, dict(o=FAKE + (2 << 30) + 64), gdn.GDN_ERR_INVALID_ARGUMENT, "overlaps"),
    ("o_aliases_state", {}, dict(o=FAKE + (5 << 30) + 256), gdn.GDN_ERR_INVALID_ARGUMENT, "overlaps"),
    ("idx_misaligned", {}, dict(idx=FAKE + (6 << 30) + 2), gdn.GDN_ERR_INVALID_ARGUMENT, "state_indices"),
]


@pytest.mark.parametrize("name,pkw,pover,status,msg", REC_CASES, ids=[c[0] for c in REC_CASES])
def test_recurrent_invalid_arguments(name, pkw, pover, status, msg):
    p = base_problem(seqlen=3, batch=4, **pkw)
    st, m = call_rec(p, **pover)
    assert st == status, (st, m)
    assert msg in m, m


def test_recurrent_slots_and_shapes():
    # without indices there must be a slot per sequence; dk != dv and any chunk are accepted
    st, m = call_rec(base_problem(seqlen=1, batch=4), num_slots=3)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "num_slots" in m
    st, m = call_rec(base_problem(seqlen=1, batch=4), num_slots=-1, idx=FAKE + (6 << 30))
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "num_slots" in m
    # a valid problem with dk != dv and chunk 32 gets past validation to the overlap check
    st, m = call_rec(base_problem(seqlen=1, batch=4, dk=128, dv=64, chunk=32), o=FAKE + 64)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "overlaps" in m


# ---- token-strided q, k, v and gradients ------------------------------------

def _bwd_strided(dq_off, dk_off, dv_off, ws_short=True):
    # q, k, v interleaved in one [T][3*H*d] buffer A, dq, dk, dv in buffer Bf at the given byte offsets
    p = base_problem(qkv_token_stride=3 * 2 * 64)
    A, Bf = FAKE, FAKE + (1 << 34)
    P = ctypes.c_void_p
    ptrs = [A, A + 256, A + 512, FAKE + (2 << 30), FAKE + (3 << 30), None, FAKE + (4 << 30), None,
            Bf + dq_off, Bf + dk_off, Bf + dv_off, FAKE + (5 << 30), FAKE + (6 << 30), None, None]
    need = gdn.lib().gdn_bwd_workspace_bytes(ctypes.byref(p))
    st = gdn.lib().gdn_bwd(ctypes.byref(p), *(P(x) if x else None for x in ptrs), P(FAKE + (1 << 38)),
                           need - 256 if ws_short else need, None)
    return st, gdn.last_error_message()


def test_strided_interleaved_outputs_are_accepted():
    # dq, dk, dv side by side in each token row share no element: the checks pass (and the
    # call then stops at the short workspace, before any launch)
    st, m = _bwd_strided(0, 256, 512)
    assert st == gdn.GDN_ERR_WORKSPACE_TOO_SMALL, m


@pytest.mark.parametrize("offs", [(0, 128, 512), (0, 256, 256 + 3 * 2 * 64 * 2 + 64), (512, 256, 608)])
def test_strided_overlapping_outputs_are_rejected(offs):
    st, m = _bwd_strided(*offs)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "overlap" in m, (offs, m)


def test_strided_output_over_an_input_is_rejected():
    p = base_problem(qkv_token_stride=3 * 2 * 64)
    P = ctypes.c_void_p
    A = FAKE
    # dq placed in the gap of buffer A that k occupies
    ptrs = [A, A + 256, A + 512, FAKE + (2 << 30), FAKE + (3 << 30), None, FAKE + (4 << 30), None,
            A + 256, FAKE + (8 << 30), FAKE + (9 << 30), FAKE + (5 << 30), FAKE + (6 << 30), None, None]
    st = gdn.lib().gdn_bwd(ctypes.byref(p), *(P(x) if x else None for x in ptrs), P(FAKE + (1 << 38)),
                           1, None)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "overlaps k" in gdn.last_error_message()


def call_fwd_noalloc(p, **over):
    ptrs, _ = fwd_ptrs(p, **over)
    P = ctypes.c_void_p
    st = gdn.lib().gdn_fwd_noalloc(ctypes.byref(p), P(ptrs["q"]), P(ptrs["k"]), P(ptrs["v"]), P(ptrs["g"]),
                                   P(ptrs["beta"]), P(ptrs["h0"]), P(ptrs["o"]), P(ptrs["ht"]), None)
    return st, gdn.last_error_message()


def test_noalloc_forward_rejects_what_the_static_scratch_cannot_hold():
    # the allocation-free forward takes its workspace from a 128 MiB static array: problems that
    # need more are rejected on the host, before any HIP call (so nothing is launched here)
    limit = 128 * 1024 * 1024
    L = gdn.lib()
    big = base_problem(seqlen=16384, heads=16)
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(big)) > limit
    st, m = call_fwd_noalloc(big)
    assert st == gdn.GDN_ERR_UNSUPPORTED and "static" in m, (st, m)
    fits = base_problem(seqlen=4096, heads=16)
    assert L.gdn_fwd_workspace_bytes(ctypes.byref(fits)) <= limit
    # argument checks are the forward's (no workspace argument)
    st, m = call_fwd_noalloc(base_problem(dk=96, dv=96))
    assert st == gdn.GDN_ERR_UNSUPPORTED, m
    st, m = call_fwd_noalloc(base_problem(), q=0)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "q is NULL" in m, m
    st, m = call_fwd_noalloc(base_problem(), o=FAKE)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT and "overlaps" in m, m
