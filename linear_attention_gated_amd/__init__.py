"""Gated DeltaNet (GDN) chunked gated delta-rule operator on AMD MI355X.

Thin Python binding of ``libgdn.so`` (C ABI declared in ``include/gdn.h``):
argument marshalling only.  Every step of the operator runs in the library's
HIP kernels; PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is missing or fails, these functions raise.

    o, ht = fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0)
    o, ht = fwd_noalloc(q, k, v, g, beta, ...)       # the same, on the library's static scratch
    dq, dk, dv, dg, dbeta, dh0 = bwd(q, k, v, g, beta, do, ...)
    o = recurrent_fwd(q, k, v, g, beta, state, state_indices=None)   # decoding, state in place
    y = gated_rmsnorm_fwd(x, z, w, eps=1e-6)          # the output gate: RMSNorm(x) w silu(z)
    dx, dz, dw = gated_rmsnorm_bwd(x, z, w, dy, eps=1e-6)
    y = causal_conv1d_fwd(x, w, bias=None, cu_seqlens=None, activation=True)   # x [B,T,C], w [C,K]
    dx, dw, dbias = causal_conv1d_bwd(x, w, dy, bias=None, cu_seqlens=None, activation=True)

Shapes: q, k [B,T,H,dk]; v [B,T,H,dv]; g, beta [B,T,H] fp32; states
[N,H,dk,dv] fp32 holding S^T.  Packed variable-length input: B = 1 and
cu_seqlens (int32, N+1) -- either one tensor (copied to host and device as
needed) or a (host_tensor, device_tensor) pair with equal contents.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARGUMENT, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE_TOO_SMALL, GDN_ERR_HIP = range(5)
GDN_F32, GDN_BF16 = 0, 1

EXPORTED = ("gdn_abi_version", "gdn_fwd_workspace_bytes", "gdn_bwd_workspace_bytes", "gdn_fwd",
            "gdn_bwd", "gdn_status_string", "gdn_last_error_message", "gdn_profile_events",
            "gdn_profile_count", "gdn_profile_name", "gdn_gated_rmsnorm_bwd_workspace_bytes",
            "gdn_gated_rmsnorm_fwd", "gdn_gated_rmsnorm_bwd", "gdn_causal_conv1d_bwd_workspace_bytes",
            "gdn_causal_conv1d_fwd", "gdn_causal_conv1d_bwd", "gdn_recurrent_fwd", "gdn_fwd_noalloc")


class GdnProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("chunk", ctypes.c_int64),
                ("num_seqs", ctypes.c_int64), ("cu_seqlens_host", ctypes.c_void_p),
                ("cu_seqlens_dev", ctypes.c_void_p), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int), ("qk_l2norm", ctypes.c_int32), ("qkv_token_stride", ctypes.c_int32)]


class GdnGatedNormProblem(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("dim", ctypes.c_int64), ("eps", ctypes.c_float),
                ("dtype", ctypes.c_int)]


class GdnConvProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("channels", ctypes.c_int64),
                ("kernel_size", ctypes.c_int64), ("num_seqs", ctypes.c_int64),
                ("cu_seqlens_host", ctypes.c_void_p), ("cu_seqlens_dev", ctypes.c_void_p),
                ("activation", ctypes.c_int32), ("dtype", ctypes.c_int)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (status_string(status), message))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build() or "
                               "python -m linear_attention_gated_amd.build" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        p, sz = ctypes.c_void_p, ctypes.c_size_t
        prob = ctypes.POINTER(GdnProblem)
        L.gdn_abi_version.restype = ctypes.c_int
        L.gdn_fwd_workspace_bytes.argtypes = [prob]
        L.gdn_fwd_workspace_bytes.restype = sz
        L.gdn_bwd_workspace_bytes.argtypes = [prob]
        L.gdn_bwd_workspace_bytes.restype = sz
        L.gdn_fwd.argtypes = [prob] + [p] * 8 + [p, sz, p]
        L.gdn_fwd.restype = ctypes.c_int
        L.gdn_fwd_noalloc.argtypes = [prob] + [p] * 8 + [p]
        L.gdn_fwd_noalloc.restype = ctypes.c_int
        L.gdn_bwd.argtypes = [prob] + [p] * 15 + [p, sz, p]
        L.gdn_bwd.restype = ctypes.c_int
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_last_error_message.restype = ctypes.c_char_p
        L.gdn_profile_events.argtypes = [ctypes.c_void_p, ctypes.c_int]
        L.gdn_profile_events.restype = ctypes.c_int
        L.gdn_profile_count.restype = ctypes.c_int
        L.gdn_profile_name.argtypes = [ctypes.c_int]
        L.gdn_profile_name.restype = ctypes.c_char_p
        gprob = ctypes.POINTER(GdnGatedNormProblem)
        L.gdn_gated_rmsnorm_bwd_workspace_bytes.argtypes = [gprob]
        L.gdn_gated_rmsnorm_bwd_workspace_bytes.restype = sz
        L.gdn_gated_rmsnorm_fwd.argtypes = [gprob] + [p] * 4 + [p]
        L.gdn_gated_rmsnorm_fwd.restype = ctypes.c_int
        L.gdn_gated_rmsnorm_bwd.argtypes = [gprob] + [p] * 7 + [p, sz, p]
        L.gdn_gated_rmsnorm_bwd.restype = ctypes.c_int
        cprob = ctypes.POINTER(GdnConvProblem)
        L.gdn_causal_conv1d_bwd_workspace_bytes.argtypes = [cprob]
        L.gdn_causal_conv1d_bwd_workspace_bytes.restype = sz
        L.gdn_causal_conv1d_fwd.argtypes = [cprob] + [p] * 4 + [p]
        L.gdn_causal_conv1d_fwd.restype = ctypes.c_int
        L.gdn_causal_conv1d_bwd.argtypes = [cprob] + [p] * 7 + [p, sz, p]
        L.gdn_causal_conv1d_bwd.restype = ctypes.c_int
        L.gdn_recurrent_fwd.argtypes = [prob] + [p] * 7 + [ctypes.c_int64, p, p]
        L.gdn_recurrent_fwd.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gdn_status_string(status).decode()


def last_error_message() -> str:
    return lib().gdn_last_error_message().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, last_error_message())


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return GDN_BF16
    if dt == torch.float32:
        return GDN_F32
    raise GdnError(GDN_ERR_UNSUPPORTED, "dtype %s (need float32 or bfloat16)" % dt)


def _cu_pair(cu_seqlens, device):
    if cu_seqlens is None:
        return None, None
    if isinstance(cu_seqlens, (tuple, list)) and len(cu_seqlens) == 2 and all(
            isinstance(x, torch.Tensor) for x in cu_seqlens):
        host, dev = cu_seqlens
    else:
        t = torch.as_tensor(cu_seqlens, dtype=torch.int32)
        host = t.cpu()
        dev = t.to(device)
    host = host.to(torch.int32).contiguous()
    dev = dev.to(torch.int32).contiguous()
    return host, dev


def make_problem(q, v, heads=None, cu_host=None, cu_dev=None, scale=1.0, qk_l2norm=False,
                 qkv_token_stride=0) -> GdnProblem:
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    p = GdnProblem()
    p.batch, p.seqlen, p.heads, p.dk, p.dv, p.chunk = B, T, H, dk, dv, 64
    p.num_seqs = 0 if cu_host is None else cu_host.numel() - 1
    p.cu_seqlens_host = None if cu_host is None else cu_host.data_ptr()
    p.cu_seqlens_dev = None if cu_dev is None else cu_dev.data_ptr()
    p.scale = float(scale)
    p.dtype = _dtype_code(q.dtype)
    p.qk_l2norm = 1 if qk_l2norm else 0
    p.qkv_token_stride = int(qkv_token_stride)
    return p


def _num_seqs(q, cu_host):
    return q.shape[0] if cu_host is None else cu_host.numel() - 1


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _qkv_stride(tensors, names, dtype, device):
    """0 when q, k, v (or their like) are all contiguous; otherwise their common token
    stride in elements: [B, T, H, d] views whose tokens are s elements apart (slices of
    one [B, T, s] buffer, e.g. a conv1d output)."""
    for t, n in zip(tensors, names):
        _require(t, n, dtype, device, contiguous=False)
    if all(t.is_contiguous() for t in tensors):
        return 0
    # The stride of a dimension of size one never moves an address (torch may report any
    # value there): with T = 1 the tokens are spaced by the batch stride, and a single
    # token (B = T = 1) has no spacing at all, which addresses like a contiguous row.
    s = None
    for t, n in zip(tensors, names):
        B, T, H, d = t.shape
        st = t.stride()
        if st[3] != 1 or (H > 1 and st[2] != d) or (B > 1 and T > 1 and st[0] != T * st[1]):
            raise ValueError("%s: a [B,T,H,d] view with rows of H*d elements, tokens evenly spaced, "
                             "is needed (strides %r)" % (n, st))
        tok = st[1] if T > 1 else (st[0] if B > 1 else None)
        if tok is None:
            continue
        if s is None:
            s = tok
        elif tok != s:
            raise ValueError("q, k and v must share one token stride (%s has %d, expected %d)" % (n, tok, s))
    return 0 if s is None else s


def _like_layout(tensors):
    """Empty tensors laid out like `tensors` (views of one storage with equal strides):
    one new buffer of the same size, viewed at the same offsets."""
    base = tensors[0]
    st = base.untyped_storage()
    for t in tensors[1:]:
        if t.untyped_storage().data_ptr() != st.data_ptr():
            raise ValueError("strided q, k, v must be views of one buffer")
    buf = torch.empty(st.nbytes() // base.element_size(), dtype=base.dtype, device=base.device)
    return [buf.as_strided(t.shape, t.stride(), t.storage_offset()) for t in tensors]


def _require(t, name, dtype, device, contiguous=True):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


class Context:
    """Forward context kept for a later backward: the forward workspace and
    the problem it was computed for."""

    def __init__(self, workspace, problem_key):
        self.workspace = workspace
        self.problem_key = problem_key


def fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0,
        output_final_state=True, return_context=False, workspace=None, qk_l2norm=False):
    """Forward pass.  Returns (o, ht) or (o, ht, Context).  With ``qk_l2norm``
    the rows of q and k are L2-normalised inside the operator."""
    dev = q.device
    dt = q.dtype
    ld = _qkv_stride((q, k, v), ("q", "k", "v"), dt, dev)
    _require(g, "g", torch.float32, dev)
    _require(beta, "beta", torch.float32, dev)
    _require(initial_state, "initial_state", torch.float32, dev)
    cu_h, cu_d = _cu_pair(cu_seqlens, dev)
    p = make_problem(q, v, cu_host=cu_h, cu_dev=cu_d, scale=scale, qk_l2norm=qk_l2norm, qkv_token_stride=ld)
    L = lib()
    nbytes = L.gdn_fwd_workspace_bytes(ctypes.byref(p))
    if nbytes == 0:
        _check(L.gdn_fwd(ctypes.byref(p), None, None, None, None, None, None, None, None, None, 0,
                         None))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    B, T, H, dk = q.shape
    N = _num_seqs(q, cu_h)
    o = torch.empty((B, T, H, v.shape[-1]), dtype=dt, device=dev)
    ht = torch.empty((N, H, dk, v.shape[-1]), dtype=torch.float32, device=dev) \
        if output_final_state else None
    _check(L.gdn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                     _ptr(initial_state), _ptr(o), _ptr(ht), _ptr(workspace), nbytes, _stream(dev)))
    if return_context:
        key = (tuple(q.shape), tuple(v.shape), dt, None if cu_h is None else tuple(cu_h.tolist()),
               float(scale), bool(qk_l2norm), ld)
        return o, ht, Context(workspace, key)
    return o, ht


def fwd_noalloc(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0,
                output_final_state=True, qk_l2norm=False, out=None, final_state=None):
    """The forward of ``fwd`` through ``gdn_fwd_noalloc``: the library allocates nothing and
    takes its workspace from its static per-GPU scratch (so no context for ``bwd``).  With
    ``out`` / ``final_state`` (preallocated o [B,T,H,dv] and ht [N,H,dk,dv]) this function
    allocates nothing either.  Returns (o, ht)."""
    dev = q.device
    dt = q.dtype
    ld = _qkv_stride((q, k, v), ("q", "k", "v"), dt, dev)
    _require(g, "g", torch.float32, dev)
    _require(beta, "beta", torch.float32, dev)
    _require(initial_state, "initial_state", torch.float32, dev)
    cu_h, cu_d = _cu_pair(cu_seqlens, dev)
    p = make_problem(q, v, cu_host=cu_h, cu_dev=cu_d, scale=scale, qk_l2norm=qk_l2norm, qkv_token_stride=ld)
    B, T, H, dk = q.shape
    N = _num_seqs(q, cu_h)
    o = out if out is not None else torch.empty((B, T, H, v.shape[-1]), dtype=dt, device=dev)
    _require(o, "out", dt, dev)
    ht = None
    if output_final_state:
        ht = final_state if final_state is not None else torch.empty((N, H, dk, v.shape[-1]), dtype=torch.float32,
                                                                     device=dev)
        _require(ht, "final_state", torch.float32, dev)
    _check(lib().gdn_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(initial_state), _ptr(o), _ptr(ht), _stream(dev)))
    return o, ht


def bwd(q, k, v, g, beta, do, initial_state=None, dht=None, cu_seqlens=None, scale=1.0,
        context: Context | None = None, need_dh0=True, workspace=None, qk_l2norm=False):
    """Backward pass of L = <do, o> + <dht, ht>.  Returns (dq, dk, dv, dg, dbeta, dh0);
    dh0 is None when need_dh0 is False.  With ``context`` from ``fwd(...,
    return_context=True)`` on the same inputs, the forward is not recomputed."""
    dev = q.device
    dt = q.dtype
    ld = _qkv_stride((q, k, v), ("q", "k", "v"), dt, dev)
    _require(do, "do", dt, dev)
    _require(g, "g", torch.float32, dev)
    _require(beta, "beta", torch.float32, dev)
    _require(initial_state, "initial_state", torch.float32, dev)
    _require(dht, "dht", torch.float32, dev)
    cu_h, cu_d = _cu_pair(cu_seqlens, dev)
    p = make_problem(q, v, cu_host=cu_h, cu_dev=cu_d, scale=scale, qk_l2norm=qk_l2norm, qkv_token_stride=ld)
    if context is not None:
        key = (tuple(q.shape), tuple(v.shape), dt, None if cu_h is None else tuple(cu_h.tolist()),
               float(scale), bool(qk_l2norm), ld)
        if key != context.problem_key:
            raise ValueError("context was computed for a different problem")
    L = lib()
    nbytes = L.gdn_bwd_workspace_bytes(ctypes.byref(p))
    if nbytes == 0:
        _check(L.gdn_bwd(ctypes.byref(p), *([None] * 16), 0, None))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    N = _num_seqs(q, cu_h)
    B, T, H, dk = q.shape
    if ld:
        # gradients laid out like the inputs: views of one new buffer
        dq, dk_, dv = _like_layout((q, k, v))
    else:
        dq = torch.empty_like(q)
        dk_ = torch.empty_like(k)
        dv = torch.empty_like(v)
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    dh0 = torch.empty((N, H, dk, v.shape[-1]), dtype=torch.float32, device=dev) if need_dh0 else None
    fws = None if context is None else context.workspace
    _check(L.gdn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                     _ptr(initial_state), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk_), _ptr(dv),
                     _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(fws), _ptr(workspace), nbytes,
                     _stream(dev)))
    return dq, dk_, dv, dg, dbeta, dh0


# ---- gated RMSNorm on the operator's output --------------------------------

GATED_NORM_EPS = 1e-6


def make_gated_norm_problem(x, eps=GATED_NORM_EPS) -> GdnGatedNormProblem:
    p = GdnGatedNormProblem()
    d = x.shape[-1] if x.dim() > 0 else 0
    p.rows = x.numel() // d if d else 0
    p.dim = d
    p.eps = float(eps)
    p.dtype = _dtype_code(x.dtype)
    return p


def gated_rmsnorm_fwd(x, z, w, eps=GATED_NORM_EPS):
    """y = x (mean(x^2) + eps)^(-1/2) w silu(z) over the last dim; x, z [..., d] in the
    problem dtype, w [d] fp32.  Returns y shaped like x."""
    dev, dt = x.device, x.dtype
    _require(x, "x", dt, dev)
    _require(z, "z", dt, dev)
    _require(w, "w", torch.float32, dev)
    if z.shape != x.shape or w.shape != (x.shape[-1],):
        raise ValueError("shapes: x %r, z %r, w %r" % (tuple(x.shape), tuple(z.shape), tuple(w.shape)))
    p = make_gated_norm_problem(x, eps)
    y = torch.empty_like(x)
    _check(lib().gdn_gated_rmsnorm_fwd(ctypes.byref(p), _ptr(x), _ptr(z), _ptr(w), _ptr(y), _stream(dev)))
    return y


def gated_rmsnorm_bwd(x, z, w, dy, eps=GATED_NORM_EPS, workspace=None):
    """Gradients (dx, dz, dw) of sum(dy * gated_rmsnorm_fwd(x, z, w, eps)); dw is fp32 [d]."""
    dev, dt = x.device, x.dtype
    for name, t in (("x", x), ("z", z), ("dy", dy)):
        _require(t, name, dt, dev)
    _require(w, "w", torch.float32, dev)
    if z.shape != x.shape or dy.shape != x.shape or w.shape != (x.shape[-1],):
        raise ValueError("shapes: x %r, z %r, dy %r, w %r"
                         % (tuple(x.shape), tuple(z.shape), tuple(dy.shape), tuple(w.shape)))
    p = make_gated_norm_problem(x, eps)
    L = lib()
    nbytes = L.gdn_gated_rmsnorm_bwd_workspace_bytes(ctypes.byref(p))
    if nbytes == 0:
        _check(L.gdn_gated_rmsnorm_bwd(ctypes.byref(p), *([None] * 8), 0, None))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dx = torch.empty_like(x)
    dz = torch.empty_like(z)
    dw = torch.empty_like(w)
    _check(L.gdn_gated_rmsnorm_bwd(ctypes.byref(p), _ptr(x), _ptr(z), _ptr(w), _ptr(dy), _ptr(dx),
                                   _ptr(dz), _ptr(dw), _ptr(workspace), nbytes, _stream(dev)))
    return dx, dz, dw


# ---- causal depthwise conv1d over packed sequences -------------------------

def make_conv_problem(x, K, cu_host=None, cu_dev=None, activation=True) -> GdnConvProblem:
    B, T, C = x.shape
    p = GdnConvProblem()
    p.batch, p.seqlen, p.channels, p.kernel_size = B, T, C, K
    p.num_seqs = 0 if cu_host is None else cu_host.numel() - 1
    p.cu_seqlens_host = None if cu_host is None else cu_host.data_ptr()
    p.cu_seqlens_dev = None if cu_dev is None else cu_dev.data_ptr()
    p.activation = 1 if activation else 0
    p.dtype = _dtype_code(x.dtype)
    return p


def _conv_args(x, w, bias, cu_seqlens):
    dev, dt = x.device, x.dtype
    _require(x, "x", dt, dev)
    _require(w, "w", torch.float32, dev)
    _require(bias, "bias", torch.float32, dev)
    if x.dim() != 3 or w.dim() != 2 or w.shape[0] != x.shape[2] or (
            bias is not None and bias.shape != (x.shape[2],)):
        raise ValueError("shapes: x %r (need [B,T,C]), w %r (need [C,K]), bias %r"
                         % (tuple(x.shape), tuple(w.shape), None if bias is None else tuple(bias.shape)))
    return _cu_pair(cu_seqlens, dev)


def causal_conv1d_fwd(x, w, bias=None, cu_seqlens=None, activation=True):
    """y[t, c] = act(bias[c] + sum_j w[c, j] x[t - (K-1) + j, c]) within each sequence;
    x [B, T, C] channels last (B = 1 with cu_seqlens), w [C, K] and bias [C] fp32."""
    cu_h, cu_d = _conv_args(x, w, bias, cu_seqlens)
    p = make_conv_problem(x, w.shape[1], cu_h, cu_d, activation)
    y = torch.empty_like(x)
    _check(lib().gdn_causal_conv1d_fwd(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(bias), _ptr(y),
                                       _stream(x.device)))
    return y


def causal_conv1d_bwd(x, w, dy, bias=None, cu_seqlens=None, activation=True, need_dbias=True,
                      workspace=None):
    """Gradients (dx, dw, dbias) of sum(dy * causal_conv1d_fwd(...)); dbias is None when
    need_dbias is False."""
    cu_h, cu_d = _conv_args(x, w, bias, cu_seqlens)
    _require(dy, "dy", x.dtype, x.device)
    if dy.shape != x.shape:
        raise ValueError("dy %r != x %r" % (tuple(dy.shape), tuple(x.shape)))
    p = make_conv_problem(x, w.shape[1], cu_h, cu_d, activation)
    L = lib()
    nbytes = L.gdn_causal_conv1d_bwd_workspace_bytes(ctypes.byref(p))
    if nbytes == 0:
        _check(L.gdn_causal_conv1d_bwd(ctypes.byref(p), *([None] * 8), 0, None))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    db = torch.empty(x.shape[2], dtype=torch.float32, device=x.device) if need_dbias else None
    _check(L.gdn_causal_conv1d_bwd(ctypes.byref(p), _ptr(x), _ptr(w), _ptr(bias), _ptr(dy), _ptr(dx),
                                   _ptr(dw), _ptr(db), _ptr(workspace), nbytes, _stream(x.device)))
    return dx, dw, db


# ---- recurrent (decoding) forward --------------------------------------------

def recurrent_fwd(q, k, v, g, beta, state, state_indices=None, cu_seqlens=None, scale=1.0,
                  qk_l2norm=False):
    """Token-by-token forward for decoding; ``state`` [num_slots, H, dk, dv] fp32 (holding
    S^T) is updated in place.  Sequence n uses slot n, or ``state_indices[n]`` (int32 on the
    device; an index outside [0, num_slots) skips the sequence and gives zero outputs).
    q, k [B, T, H, dk], v [B, T, H, dv] (B = 1 with cu_seqlens); dk and dv may differ.
    Returns o [B, T, H, dv]."""
    dev, dt = q.device, q.dtype
    ld = _qkv_stride((q, k, v), ("q", "k", "v"), dt, dev)
    _require(g, "g", torch.float32, dev)
    _require(beta, "beta", torch.float32, dev)
    _require(state, "state", torch.float32, dev)
    _require(state_indices, "state_indices", torch.int32, dev)
    cu_h, cu_d = _cu_pair(cu_seqlens, dev)
    p = make_problem(q, v, cu_host=cu_h, cu_dev=cu_d, scale=scale, qk_l2norm=qk_l2norm, qkv_token_stride=ld)
    o = torch.empty(v.shape, dtype=dt, device=dev)
    _check(lib().gdn_recurrent_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(state), _ptr(state_indices), state.shape[0], _ptr(o), _stream(dev)))
    return o
