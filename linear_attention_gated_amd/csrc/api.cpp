// api.cpp -- the C ABI of libgdn.so: argument validation, workspace layout
// and the launch sequence.  Every check runs on the host before any HIP call.
//
// Launch sequence (all on the caller's stream, no host synchronisation):
//   forward : plan -> K1 prep (gamma, T = (I+A)^-1, WY factors)
//                  -> K2 state pass (sequential over chunks)
//                  -> K3 output
//   backward: [plan -> K1 -> K2 recompute, unless a forward workspace is given]
//             -> K4 prep -> K5 reverse state-gradient pass -> K6 gradients
// The split mirrors the native kernel family of the XTuner / Ascend 910C
// article (section 3.1.2, Fig. 7): a forward state update that also runs
// inside the backward, the reverse pass through the state-transition chain,
// the local dv step and the dq/dk/dw/dg step.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

// Optional per-launch event bracketing (timing diagnostics), per thread.
struct ProfileState {
  void* const* events = nullptr;
  int pairs = 0;
  int count = 0;
  const char* names[512] = {};
};
thread_local ProfileState g_prof;

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& f) {
  ProfileState& P = g_prof;
  const bool rec = P.events && P.count < P.pairs;
  if (rec) {
    hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(P.events[2 * P.count]), s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = f();
  if (rec) {
    hipError_t e2 = hipEventRecord(reinterpret_cast<hipEvent_t>(P.events[2 * P.count + 1]), s);
    if (P.count < 512) P.names[P.count] = name;
    ++P.count;
    if (e == hipSuccess) e = e2;
  }
  return e;
}

gdn_status fail(gdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

// The dtype field as the integer the caller stored: a C caller may put any
// int in the enum, and loading an out-of-range value through the enum type
// itself would be undefined in C++.
template <class Prob>
int dtype_of(const Prob* p) {
  int v;
  static_assert(sizeof(v) == sizeof(p->dtype), "the dtype field is an int");
  std::memcpy(&v, &p->dtype, sizeof(v));
  return v;
}

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Token stride (elements) of q, k, v and their gradients: 0 means contiguous.
gdn_status check_stride(const gdn_problem* p) {
  const int64_t s = p->qkv_token_stride;
  if (s == 0) return GDN_OK;
  const int64_t wmax = p->heads * (p->dk > p->dv ? p->dk : p->dv);
  const int64_t mult = dtype_of(p) == GDN_BF16 ? 8 : 4;
  if (s < 0 || s < wmax)
    return fail(GDN_ERR_INVALID_ARGUMENT, "qkv_token_stride %lld < H * max(dk, dv) = %lld", (long long)s, (long long)wmax);
  if (s % mult) return fail(GDN_ERR_INVALID_ARGUMENT, "qkv_token_stride %lld is not a multiple of %lld", (long long)s, (long long)mult);
  return GDN_OK;
}

// Memory of a [tokens][width] tensor whose tokens are `stride` elements apart
// (bytes from p): rows [p + t * stride * esz, + width * esz).
struct Strided {
  const void* p;
  int64_t tokens, width, stride;   // elements
  size_t esz;
  const char* name;
  size_t span() const { return tokens > 0 ? (size_t)((tokens - 1) * stride + width) * esz : 0; }
};

// Do two tensors share a byte?  Same stride: some rows r1, r2 of A and B
// intersect, i.e. -wb < d + k * S < wa for d = pB - pA and some k = r2 - r1
// with |k| < tokens; otherwise (or for contiguous tensors) by their spans.
bool strided_overlap(const Strided& a, const Strided& b) {
  if (!a.p || !b.p || a.span() == 0 || b.span() == 0) return false;
  const long long pa = (long long)(uintptr_t)a.p, pb = (long long)(uintptr_t)b.p;
  const long long wa = a.width * (long long)a.esz, wb = b.width * (long long)b.esz;
  if (a.stride == b.stride && a.esz == b.esz && a.stride > a.width && b.stride > b.width && a.tokens == b.tokens) {
    const long long S = a.stride * (long long)a.esz, d = pb - pa, T = a.tokens;
    // integers k with (-wb - d) / S < k < (wa - d) / S
    auto fdiv = [](long long x, long long y) { return x / y - ((x % y != 0) && ((x < 0) != (y < 0))); };
    const long long klo = fdiv(-wb - d, S) + 1, khi = -fdiv(-(wa - d), S) - 1;
    const long long lo = klo > -(T - 1) ? klo : -(T - 1), hi = khi < T - 1 ? khi : T - 1;
    return lo <= hi;
  }
  return pa < pb + (long long)b.span() && pb < pa + (long long)a.span();
}

struct Layout {
  int64_t B = 0, T = 0, H = 0, N = 0, NC = 0, tokens = 0;
  int64_t DK = 0, DV = 0, D = 0;   // head dims; the kernels run at D = max(DK, DV)
  bool varlen = false, bf16 = false, l2norm = false;
  size_t esz = 0;
  int64_t ldq = 0, ldv = 0;   // token strides (elements) of q, k, dq, dk and of v, dv
  // byte offsets into a workspace
  size_t chunk_tab = 0, seq_tab = 0, gamma = 0, Wn = 0, Ktf = 0, Ua = 0, Hf = 0, Vf = 0, Tm = 0;
  size_t qinv = 0, kinv = 0;
  size_t fwd_bytes = 0;
  size_t Z = 0, WnT = 0, Ktn = 0, HPf = 0, dVf = 0, dVl = 0;
  size_t bwd_bytes = 0;
};

// Validate the problem description and derive sizes.  No HIP call.
gdn_status plan_problem(const gdn_problem* p, Layout* L) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (dtype_of(p) != GDN_F32 && dtype_of(p) != GDN_BF16)
    return fail(GDN_ERR_UNSUPPORTED, "dtype %d is not GDN_F32 or GDN_BF16", dtype_of(p));
  if (p->heads < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "heads = %lld < 1", (long long)p->heads);
  if (p->dk < 1 || p->dv < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "dk/dv must be >= 1");
  if ((p->dk != 64 && p->dk != 128) || (p->dv != 64 && p->dv != 128))
    return fail(GDN_ERR_UNSUPPORTED, "head dims dk %lld, dv %lld not in {64, 128}", (long long)p->dk, (long long)p->dv);
  if (p->chunk != 64) return fail(GDN_ERR_UNSUPPORTED, "chunk %lld != 64", (long long)p->chunk);
  if (!std::isfinite(p->scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (p->qk_l2norm != 0 && p->qk_l2norm != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "qk_l2norm = %d is not 0 or 1", (int)p->qk_l2norm);
  if (p->seqlen < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "seqlen < 0");
  {
    gdn_status st = check_stride(p);
    if (st != GDN_OK) return st;
  }
  const bool has_h = p->cu_seqlens_host != nullptr, has_d = p->cu_seqlens_dev != nullptr;
  if (has_h != has_d)
    return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens_host and cu_seqlens_dev must both be set or both be NULL");
  L->varlen = has_h;
  L->H = p->heads;
  L->DK = p->dk;
  L->DV = p->dv;
  L->D = p->dk > p->dv ? p->dk : p->dv;
  L->T = p->seqlen;
  L->bf16 = dtype_of(p) == GDN_BF16;
  L->l2norm = p->qk_l2norm == 1;
  L->esz = L->bf16 ? 2 : 4;
  L->ldq = p->qkv_token_stride ? p->qkv_token_stride : p->heads * p->dk;
  L->ldv = p->qkv_token_stride ? p->qkv_token_stride : p->heads * p->dv;
  const int64_t maxtok = (int64_t)1 << 31;
  if (L->varlen) {
    if (p->batch != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "varlen requires batch == 1 (got %lld)", (long long)p->batch);
    if (p->num_seqs < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs = %lld < 1", (long long)p->num_seqs);
    if (((uintptr_t)p->cu_seqlens_dev) % 4) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens_dev misaligned");
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[0] = %d != 0", cu[0]);
    int64_t nc = 0;
    for (int64_t n = 0; n < p->num_seqs; ++n) {
      if (cu[n + 1] < cu[n])
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %lld (%d -> %d)", (long long)n, cu[n], cu[n + 1]);
      nc += (cu[n + 1] - cu[n] + 63) / 64;
    }
    if (cu[p->num_seqs] != p->seqlen)
      return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[N] = %d != seqlen %lld", cu[p->num_seqs], (long long)p->seqlen);
    L->B = 1;
    L->N = p->num_seqs;
    L->NC = nc;
  } else {
    if (p->batch < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "batch = %lld < 1", (long long)p->batch);
    L->B = p->batch;
    L->N = p->batch;
    L->NC = p->batch * ((p->seqlen + 63) / 64);
  }
  L->tokens = L->B * L->T;
  if (L->tokens * L->H >= maxtok || L->NC * L->H >= maxtok / 64 || L->N * L->H >= maxtok / 64)
    return fail(GDN_ERR_UNSUPPORTED, "problem too large (tokens*heads must stay below 2^31)");

  // workspace layout
  const size_t ch = (size_t)(L->NC * L->H);
  const size_t D = (size_t)L->D, e = L->esz;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L->chunk_tab = take(sizeof(int32_t) * 4 * (size_t)L->NC);
  L->seq_tab = take(sizeof(int32_t) * 4 * (size_t)L->N);
  L->gamma = take(sizeof(float) * 64 * ch);
  L->Wn = take(e * ch * 64 * D);
  L->Ktf = take(e * ch * 64 * D);
  L->Ua = take(e * ch * 64 * D);
  L->Hf = take(e * ch * D * D);
  L->Vf = take(e * ch * 64 * D);
  L->Tm = take(sizeof(float) * ch * 64 * 64);
  if (L->l2norm) L->kinv = take(sizeof(float) * (size_t)(L->tokens * L->H));
  L->fwd_bytes = off;
  L->Z = take(e * ch * D * D);
  L->WnT = take(e * ch * 64 * D);
  L->Ktn = take(e * ch * 64 * D);
  L->HPf = take(e * ch * D * D);
  L->dVf = take(e * ch * 64 * D);
  L->dVl = take(e * ch * 64 * D);
  if (L->l2norm) L->qinv = take(sizeof(float) * (size_t)(L->tokens * L->H));
  L->bwd_bytes = off;
  return GDN_OK;
}

// A buffer: n bytes from p, or, with a token stride, `tokens` rows of `width`
// elements `stride` elements apart (n is then the span).
struct Range {
  const void* p;
  size_t n;
  const char* name;
  int64_t tokens = 0, width = 0, stride = 0;
  size_t esz = 0;
};

Range strided(const void* p, int64_t tokens, int64_t width, int64_t stride, size_t esz, const char* name) {
  Range r{p, tokens > 0 ? (size_t)((tokens - 1) * stride + width) * esz : 0, name};
  r.tokens = tokens;
  r.width = width;
  r.stride = stride;
  r.esz = esz;
  return r;
}

bool overlaps(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  if (a.stride && b.stride)
    return strided_overlap({a.p, a.tokens, a.width, a.stride, a.esz, a.name},
                           {b.p, b.tokens, b.width, b.stride, b.esz, b.name});
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

gdn_status check_ptrs(const Range* req, int nreq, const Range* opt, int nopt, const Range* outs, int nout,
                      const Range* ins, int nin) {
  for (int i = 0; i < nreq; ++i) {
    if (req[i].n > 0 && !req[i].p) return fail(GDN_ERR_INVALID_ARGUMENT, "%s is NULL", req[i].name);
  }
  for (int i = 0; i < nreq + nopt; ++i) {
    const Range& r = i < nreq ? req[i] : opt[i - nreq];
    if (r.p && ((uintptr_t)r.p) % 16)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", r.name);
  }
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j]))
        return fail(GDN_ERR_INVALID_ARGUMENT, "output %s overlaps %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j]))
        return fail(GDN_ERR_INVALID_ARGUMENT, "outputs %s and %s overlap", outs[i].name, outs[j].name);
  }
  return GDN_OK;
}

// Device that work enqueued on stream s runs on (the null stream: the
// calling thread's current device).
hipError_t stream_device(hipStream_t s, int* dev) {
  return s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev);
}

// Compute units of the device of stream s, cached per device (256 on a whole
// MI355X; fewer when the GPU is partitioned).
int device_cus(hipStream_t s) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (stream_device(s, &dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

gdn::Params base_params(const gdn_problem* p, const Layout& L, char* ws, hipStream_t s) {
  gdn::Params P;
  std::memset(&P, 0, sizeof(P));
  P.H = (int)L.H;
  P.N = (int)L.N;
  P.NC = (int)L.NC;
  P.scale = p->scale;
  P.dense_T = L.varlen ? 0 : (int)L.T;
  P.total_tokens = (int)L.tokens;
  P.cu = L.varlen ? p->cu_seqlens_dev : nullptr;
  P.chunk_tab = reinterpret_cast<int4*>(ws + L.chunk_tab);
  P.seq_tab = reinterpret_cast<int4*>(ws + L.seq_tab);
  P.gamma = reinterpret_cast<float*>(ws + L.gamma);
  P.Wn = ws + L.Wn;
  P.Ktf = ws + L.Ktf;
  P.Ua = ws + L.Ua;
  P.Hf = ws + L.Hf;
  P.Vf = ws + L.Vf;
  P.Tm = reinterpret_cast<float*>(ws + L.Tm);
  P.qk_l2norm = L.l2norm ? 1 : 0;
  P.kdim = (int)L.DK;
  P.vdim = (int)L.DV;
  P.ldq = L.ldq;
  P.ldv = L.ldv;
  // State-pass workgroups, one per (sequence, head, 16-column block), one
  // resident per CU: with more than half the CUs' worth, rotated shared reads
  // (measured 8-11% faster there, 1-2% slower with fewer); with more than one
  // round's worth, two column blocks per workgroup (24% faster at twice the
  // CUs, 4-18% slower at one round).
  const int64_t state_wgs = L.N * L.H * (L.D / 16), cus = device_cus(s);
  P.dma_rot = state_wgs > cus / 2 ? 1 : 0;
  P.state_cpw = state_wgs > cus ? 2 : 1;
  // k_bwd_grad holds one workgroup per CU (bf16, d = 128): a round is one
  // workgroup per CU, and workgroups `cus` apart share an XCD when it is a
  // multiple of 8
  P.grad_ahead = (int)(cus / 8 * 8);
  if (L.l2norm) P.kinv = reinterpret_cast<float*>(ws + L.kinv);
  return P;
}

gdn_status hip_fail(hipError_t e, const char* what) {
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

gdn_status check_gnorm(const gdn_gated_norm_problem* p) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (dtype_of(p) != GDN_F32 && dtype_of(p) != GDN_BF16)
    return fail(GDN_ERR_INVALID_ARGUMENT, "dtype %d is not GDN_F32 or GDN_BF16", dtype_of(p));
  if (p->rows < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "rows < 0");
  if (p->dim != 64 && p->dim != 128) return fail(GDN_ERR_UNSUPPORTED, "dim %lld not in {64, 128}", (long long)p->dim);
  if (!std::isfinite(p->eps) || p->eps < 0.f) return fail(GDN_ERR_INVALID_ARGUMENT, "eps is negative or not finite");
  if (p->rows > ((int64_t)1 << 40) / p->dim) return fail(GDN_ERR_UNSUPPORTED, "problem too large");
  return GDN_OK;
}

struct ConvPlan {
  int64_t tokens = 0, N = 0, T = 0;
  bool varlen = false, bf16 = false;
};

gdn_status check_conv(const gdn_conv_problem* p, ConvPlan* P) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (dtype_of(p) != GDN_F32 && dtype_of(p) != GDN_BF16)
    return fail(GDN_ERR_UNSUPPORTED, "dtype %d is not GDN_F32 or GDN_BF16", dtype_of(p));
  if (p->kernel_size < 1 || p->kernel_size > 4)
    return fail(GDN_ERR_UNSUPPORTED, "kernel_size %lld not in [1, 4]", (long long)p->kernel_size);
  if (p->channels < 1 || p->channels % 4)
    return fail(GDN_ERR_UNSUPPORTED, "channels %lld is not a positive multiple of 4", (long long)p->channels);
  if (p->activation != 0 && p->activation != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "activation = %d is not 0 or 1", (int)p->activation);
  if (p->seqlen < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "seqlen < 0");
  const bool has_h = p->cu_seqlens_host != nullptr, has_d = p->cu_seqlens_dev != nullptr;
  if (has_h != has_d)
    return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens_host and cu_seqlens_dev must both be set or both be NULL");
  P->varlen = has_h;
  P->bf16 = dtype_of(p) == GDN_BF16;
  P->T = p->seqlen;
  if (P->varlen) {
    if (p->batch != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "varlen requires batch == 1 (got %lld)", (long long)p->batch);
    if (p->num_seqs < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs = %lld < 1", (long long)p->num_seqs);
    if (((uintptr_t)p->cu_seqlens_dev) % 4) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens_dev misaligned");
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[0] = %d != 0", cu[0]);
    for (int64_t n = 0; n < p->num_seqs; ++n)
      if (cu[n + 1] < cu[n])
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %lld (%d -> %d)", (long long)n, cu[n], cu[n + 1]);
    if (cu[p->num_seqs] != p->seqlen)
      return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[N] = %d != seqlen %lld", cu[p->num_seqs], (long long)p->seqlen);
    P->N = p->num_seqs;
  } else {
    if (p->batch < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "batch = %lld < 1", (long long)p->batch);
    P->N = p->batch;
  }
  P->tokens = (P->varlen ? 1 : p->batch) * p->seqlen;
  if (P->tokens >= ((int64_t)1 << 31) || P->N >= ((int64_t)1 << 31) ||
      P->tokens * p->channels >= ((int64_t)1 << 40))
    return fail(GDN_ERR_UNSUPPORTED, "problem too large");
  return GDN_OK;
}

size_t conv_ws_bytes(const gdn_conv_problem* p, const ConvPlan& P) {
  const int rows = gdn::conv_bwd_rows(P.tokens, (int)p->channels);
  return align_up((size_t)(rows > 0 ? rows : 1) * (size_t)p->channels * (size_t)(p->kernel_size + 1) * sizeof(float));
}

gdn::ConvParams conv_params(const gdn_conv_problem* p, const ConvPlan& P) {
  gdn::ConvParams c;
  std::memset(&c, 0, sizeof(c));
  c.cu = P.varlen ? p->cu_seqlens_dev : nullptr;
  c.N = (int)P.N;
  c.dense_T = P.varlen ? 0 : (int)P.T;
  c.tokens = P.tokens;
  c.C = (int)p->channels;
  c.K = (int)p->kernel_size;
  c.act = p->activation;
  return c;
}

struct RecPlan {
  int64_t tokens = 0, N = 0;
  bool varlen = false, bf16 = false;
};

gdn_status check_recurrent(const gdn_problem* p, RecPlan* P) {
  if (!p) return fail(GDN_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (dtype_of(p) != GDN_F32 && dtype_of(p) != GDN_BF16)
    return fail(GDN_ERR_UNSUPPORTED, "dtype %d is not GDN_F32 or GDN_BF16", dtype_of(p));
  if (p->heads < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "heads = %lld < 1", (long long)p->heads);
  if ((p->dk != 64 && p->dk != 128) || (p->dv != 64 && p->dv != 128))
    return fail(GDN_ERR_UNSUPPORTED, "dk %lld / dv %lld not in {64, 128}", (long long)p->dk, (long long)p->dv);
  if (!std::isfinite(p->scale)) return fail(GDN_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (p->qk_l2norm != 0 && p->qk_l2norm != 1)
    return fail(GDN_ERR_INVALID_ARGUMENT, "qk_l2norm = %d is not 0 or 1", (int)p->qk_l2norm);
  if (p->seqlen < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "seqlen < 0");
  {
    gdn_status st = check_stride(p);
    if (st != GDN_OK) return st;
  }
  const bool has_h = p->cu_seqlens_host != nullptr, has_d = p->cu_seqlens_dev != nullptr;
  if (has_h != has_d)
    return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens_host and cu_seqlens_dev must both be set or both be NULL");
  P->varlen = has_h;
  P->bf16 = dtype_of(p) == GDN_BF16;
  if (P->varlen) {
    if (p->batch != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "varlen requires batch == 1 (got %lld)", (long long)p->batch);
    if (p->num_seqs < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "num_seqs = %lld < 1", (long long)p->num_seqs);
    if (((uintptr_t)p->cu_seqlens_dev) % 4) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens_dev misaligned");
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0) return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[0] = %d != 0", cu[0]);
    for (int64_t n = 0; n < p->num_seqs; ++n)
      if (cu[n + 1] < cu[n])
        return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens decreases at %lld (%d -> %d)", (long long)n, cu[n], cu[n + 1]);
    if (cu[p->num_seqs] != p->seqlen)
      return fail(GDN_ERR_INVALID_ARGUMENT, "cu_seqlens[N] = %d != seqlen %lld", cu[p->num_seqs], (long long)p->seqlen);
    P->N = p->num_seqs;
  } else {
    if (p->batch < 1) return fail(GDN_ERR_INVALID_ARGUMENT, "batch = %lld < 1", (long long)p->batch);
    P->N = p->batch;
  }
  P->tokens = (P->varlen ? 1 : p->batch) * p->seqlen;
  if (P->tokens * p->heads >= ((int64_t)1 << 31) || P->N * p->heads >= ((int64_t)1 << 31))
    return fail(GDN_ERR_UNSUPPORTED, "problem too large");
  return GDN_OK;
}

size_t gnorm_ws_bytes(const gdn_gated_norm_problem* p) {
  const int nb = gdn::gnorm_blocks(p->rows, (int)p->dim, dtype_of(p) == GDN_BF16, true);
  return align_up((size_t)(nb > 0 ? nb : 1) * (size_t)p->dim * sizeof(float));
}

// Forward arguments; with_ws: a caller workspace of L.fwd_bytes is required
// (gdn_fwd), without it none is passed (gdn_fwd_noalloc).
gdn_status check_fwd_args(const Layout& L, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* h0, const void* o, const float* ht,
                          const void* workspace, bool with_ws) {
  const size_t ob = (size_t)(L.tokens * L.H * L.DV) * L.esz;
  const size_t gb = (size_t)(L.tokens * L.H) * sizeof(float);
  const size_t sb = (size_t)(L.N * L.H * L.DK * L.DV) * sizeof(float);
  const Range rq = strided(q, L.tokens, L.H * L.DK, L.ldq, L.esz, "q"), rk = strided(k, L.tokens, L.H * L.DK, L.ldq, L.esz, "k"),
              rv = strided(v, L.tokens, L.H * L.DV, L.ldv, L.esz, "v");
  const size_t wb = with_ws ? L.fwd_bytes : 0;
  const Range req[] = {rq, rk, rv, {g, gb, "g"}, {beta, gb, "beta"}, {o, ob, "o"}, {workspace, wb, "workspace"}};
  const Range opt[] = {{h0, sb, "h0"}, {ht, sb, "ht"}};
  const Range outs[] = {{o, ob, "o"}, {ht, sb, "ht"}, {workspace, wb, "workspace"}};
  const Range ins[] = {rq, rk, rv, {g, gb, "g"}, {beta, gb, "beta"}, {h0, sb, "h0"}};
  return check_ptrs(req, with_ws ? 7 : 6, opt, 2, outs, 3, ins, 6);
}

// The forward's launch sequence on stream s, with its workspace at ws.
gdn_status fwd_launch(const gdn_problem* p, const Layout& L, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const float* h0, void* o, float* ht, char* ws,
                      hipStream_t s) {
  gdn::Params P = base_params(p, L, ws, s);
  P.q = q; P.k = k; P.v = v; P.g = g; P.beta = beta; P.h0 = h0; P.o = o; P.ht = ht;
  const int D = (int)L.D;
  hipError_t e;
  // (packed input only: for dense input the chunk tables are arithmetic and nothing is launched)
  if (L.varlen && (e = timed("plan", s, [&] { return gdn::launch_plan(P, s); })) != hipSuccess) return hip_fail(e, "plan launch");
  if ((e = timed("fwd_prep", s, [&] { return gdn::launch_fwd_prep(P, D, L.bf16, s); })) != hipSuccess) return hip_fail(e, "fwd_prep launch");
  if ((e = timed("fwd_state", s, [&] { return gdn::launch_fwd_state(P, D, L.bf16, true, s); })) != hipSuccess) return hip_fail(e, "fwd_state launch");
  if ((e = timed("fwd_out", s, [&] { return gdn::launch_fwd_out(P, D, L.bf16, s); })) != hipSuccess) return hip_fail(e, "fwd_out launch");
  return GDN_OK;
}

}  // namespace

// Scratch of gdn_fwd_noalloc: a static device array, one copy on every GPU the
// library runs on, held until the process ends.  In host code `scratch`
// names a host-side stand-in; its device address on each GPU is looked up
// once (hipGetSymbolAddress, with that GPU current) and only that address is
// handed to kernels.
static __device__ __align__(256) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
char* g_scratch_dev[64] = {};

// Device address of GPU dev's copy of `scratch`.
hipError_t static_scratch(int dev, char** out) {
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!ptr || ((uintptr_t)ptr) % ALIGN) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = reinterpret_cast<char*>(ptr);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "GDN_ERR_WORKSPACE_TOO_SMALL";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
  }
  return "GDN_ERR_UNKNOWN";
}

const char* gdn_last_error_message(void) { return g_last_error.c_str(); }

size_t gdn_gated_rmsnorm_bwd_workspace_bytes(const gdn_gated_norm_problem* p) {
  try {
    if (check_gnorm(p) != GDN_OK) return 0;
    return gnorm_ws_bytes(p);
  } catch (...) {
    return 0;
  }
}

gdn_status gdn_gated_rmsnorm_fwd(const gdn_gated_norm_problem* p, const void* x, const void* z,
                                 const float* w, void* y, void* stream) {
  try {
    gdn_status st = check_gnorm(p);
    if (st != GDN_OK) return st;
    const size_t rb = (size_t)(p->rows * p->dim) * (dtype_of(p) == GDN_BF16 ? 2 : 4);
    const size_t wb = (size_t)p->dim * sizeof(float);
    const Range req[] = {{x, rb, "x"}, {z, rb, "z"}, {w, wb, "w"}, {y, rb, "y"}};
    const Range outs[] = {{y, rb, "y"}};
    const Range ins[] = {{x, rb, "x"}, {z, rb, "z"}, {w, wb, "w"}};
    st = check_ptrs(req, 4, nullptr, 0, outs, 1, ins, 3);
    if (st != GDN_OK) return st;
    gdn::GnormParams P;
    std::memset(&P, 0, sizeof(P));
    P.x = x; P.z = z; P.w = w; P.y = y; P.rows = p->rows; P.eps = p->eps;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = timed("gnorm_fwd", s, [&] { return gdn::launch_gnorm_fwd(P, (int)p->dim, dtype_of(p) == GDN_BF16, s); });
    if (e != hipSuccess) return hip_fail(e, "gated rmsnorm forward launch");
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "unexpected exception in gdn_gated_rmsnorm_fwd");
  }
}

gdn_status gdn_gated_rmsnorm_bwd(const gdn_gated_norm_problem* p, const void* x, const void* z,
                                 const float* w, const void* dy, void* dx, void* dz, float* dw,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  try {
    gdn_status st = check_gnorm(p);
    if (st != GDN_OK) return st;
    const size_t rb = (size_t)(p->rows * p->dim) * (dtype_of(p) == GDN_BF16 ? 2 : 4);
    const size_t wb = (size_t)p->dim * sizeof(float);
    const size_t need = gnorm_ws_bytes(p);
    const Range req[] = {{x, rb, "x"}, {z, rb, "z"}, {w, wb, "w"}, {dy, rb, "dy"}, {dx, rb, "dx"},
                         {dz, rb, "dz"}, {dw, wb, "dw"}, {workspace, need, "workspace"}};
    const Range outs[] = {{dx, rb, "dx"}, {dz, rb, "dz"}, {dw, wb, "dw"}, {workspace, need, "workspace"}};
    const Range ins[] = {{x, rb, "x"}, {z, rb, "z"}, {w, wb, "w"}, {dy, rb, "dy"}};
    st = check_ptrs(req, 8, nullptr, 0, outs, 4, ins, 4);
    if (st != GDN_OK) return st;
    if (workspace && ((uintptr_t)workspace) % ALIGN)
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    gdn::GnormParams P;
    std::memset(&P, 0, sizeof(P));
    P.x = x; P.z = z; P.w = w; P.dy = dy; P.dx = dx; P.dz = dz; P.dw = dw;
    P.part = reinterpret_cast<float*>(workspace);
    P.rows = p->rows; P.eps = p->eps;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = timed("gnorm_bwd", s, [&] { return gdn::launch_gnorm_bwd(P, (int)p->dim, dtype_of(p) == GDN_BF16, s); });
    if (e != hipSuccess) return hip_fail(e, "gated rmsnorm backward launch");
    e = timed("gnorm_dw", s, [&] { return gdn::launch_gnorm_dw(P, (int)p->dim, dtype_of(p) == GDN_BF16, s); });
    if (e != hipSuccess) return hip_fail(e, "gated rmsnorm weight-gradient launch");
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "unexpected exception in gdn_gated_rmsnorm_bwd");
  }
}

size_t gdn_causal_conv1d_bwd_workspace_bytes(const gdn_conv_problem* p) {
  try {
    ConvPlan P;
    if (check_conv(p, &P) != GDN_OK) return 0;
    return conv_ws_bytes(p, P);
  } catch (...) {
    return 0;
  }
}

gdn_status gdn_causal_conv1d_fwd(const gdn_conv_problem* p, const void* x, const float* w,
                                 const float* bias, void* y, void* stream) {
  try {
    ConvPlan P;
    gdn_status st = check_conv(p, &P);
    if (st != GDN_OK) return st;
    const size_t xb = (size_t)(P.tokens * p->channels) * (P.bf16 ? 2 : 4);
    const size_t wb = (size_t)(p->channels * p->kernel_size) * sizeof(float);
    const size_t bb = (size_t)p->channels * sizeof(float);
    const Range req[] = {{x, xb, "x"}, {w, wb, "w"}, {y, xb, "y"}};
    const Range opt[] = {{bias, bb, "bias"}};
    const Range outs[] = {{y, xb, "y"}};
    const Range ins[] = {{x, xb, "x"}, {w, wb, "w"}, {bias, bb, "bias"}};
    st = check_ptrs(req, 3, opt, 1, outs, 1, ins, 3);
    if (st != GDN_OK) return st;
    gdn::ConvParams c = conv_params(p, P);
    c.x = x; c.w = w; c.bias = bias; c.y = y;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = timed("conv_fwd", s, [&] { return gdn::launch_conv_fwd(c, P.bf16, s); });
    if (e != hipSuccess) return hip_fail(e, "causal conv1d forward launch");
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "unexpected exception in gdn_causal_conv1d_fwd");
  }
}

gdn_status gdn_causal_conv1d_bwd(const gdn_conv_problem* p, const void* x, const float* w,
                                 const float* bias, const void* dy, void* dx, float* dw,
                                 float* dbias, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  try {
    ConvPlan P;
    gdn_status st = check_conv(p, &P);
    if (st != GDN_OK) return st;
    const size_t xb = (size_t)(P.tokens * p->channels) * (P.bf16 ? 2 : 4);
    const size_t wb = (size_t)(p->channels * p->kernel_size) * sizeof(float);
    const size_t bb = (size_t)p->channels * sizeof(float);
    const size_t need = conv_ws_bytes(p, P);
    const Range req[] = {{x, xb, "x"}, {w, wb, "w"}, {dy, xb, "dy"}, {dx, xb, "dx"}, {dw, wb, "dw"},
                         {workspace, need, "workspace"}};
    const Range opt[] = {{bias, bb, "bias"}, {dbias, bb, "dbias"}};
    const Range outs[] = {{dx, xb, "dx"}, {dw, wb, "dw"}, {dbias, bb, "dbias"}, {workspace, need, "workspace"}};
    const Range ins[] = {{x, xb, "x"}, {w, wb, "w"}, {bias, bb, "bias"}, {dy, xb, "dy"}};
    st = check_ptrs(req, 6, opt, 2, outs, 4, ins, 4);
    if (st != GDN_OK) return st;
    if (workspace && ((uintptr_t)workspace) % ALIGN)
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
    gdn::ConvParams c = conv_params(p, P);
    c.x = x; c.w = w; c.bias = bias; c.dy = dy; c.dx = dx; c.dw = dw; c.dbias = dbias;
    c.part = reinterpret_cast<float*>(workspace);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = timed("conv_bwd", s, [&] { return gdn::launch_conv_bwd(c, P.bf16, s); });
    if (e != hipSuccess) return hip_fail(e, "causal conv1d backward launch");
    e = timed("conv_dw", s, [&] { return gdn::launch_conv_dw(c, s); });
    if (e != hipSuccess) return hip_fail(e, "causal conv1d weight-gradient launch");
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "unexpected exception in gdn_causal_conv1d_bwd");
  }
}

gdn_status gdn_recurrent_fwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, float* state,
                             const int32_t* state_indices, int64_t num_slots, void* o,
                             void* stream) {
  try {
    RecPlan P;
    gdn_status st = check_recurrent(p, &P);
    if (st != GDN_OK) return st;
    if (num_slots < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "num_slots < 0");
    if (!state_indices && num_slots < P.N)
      return fail(GDN_ERR_INVALID_ARGUMENT, "num_slots %lld < %lld sequences without state_indices",
                  (long long)num_slots, (long long)P.N);
    if (state_indices && ((uintptr_t)state_indices) % 4)
      return fail(GDN_ERR_INVALID_ARGUMENT, "state_indices misaligned");
    const size_t e = P.bf16 ? 2 : 4;
    const size_t vb = (size_t)(P.tokens * p->heads * p->dv) * e;
    const size_t gb = (size_t)(P.tokens * p->heads) * sizeof(float);
    const size_t sb = (size_t)num_slots * (size_t)(p->heads * p->dk * p->dv) * sizeof(float);
    const size_t ib = state_indices ? (size_t)P.N * sizeof(int32_t) : 0;
    const int64_t ldq = p->qkv_token_stride ? p->qkv_token_stride : p->heads * p->dk;
    const int64_t ldv = p->qkv_token_stride ? p->qkv_token_stride : p->heads * p->dv;
    const Range rq = strided(q, P.tokens, p->heads * p->dk, ldq, e, "q"), rk = strided(k, P.tokens, p->heads * p->dk, ldq, e, "k"),
                rv = strided(v, P.tokens, p->heads * p->dv, ldv, e, "v");
    const Range req[] = {rq, rk, rv, {g, gb, "g"}, {beta, gb, "beta"},
                         {o, vb, "o"}, {state, P.N > 0 && num_slots > 0 ? sb : 0, "state"}};
    const Range outs[] = {{o, vb, "o"}};
    const Range ins[] = {rq, rk, rv, {g, gb, "g"}, {beta, gb, "beta"},
                         {state, sb, "state"}, {state_indices, ib, "state_indices"}};
    st = check_ptrs(req, 7, nullptr, 0, outs, 1, ins, 7);
    if (st != GDN_OK) return st;
    if (state_indices && overlaps({state_indices, ib, "state_indices"}, {state, sb, "state"}))
      return fail(GDN_ERR_INVALID_ARGUMENT, "state_indices overlaps state");
    gdn::RecParams R;
    std::memset(&R, 0, sizeof(R));
    R.q = q; R.k = k; R.v = v; R.g = g; R.beta = beta; R.state = state; R.idx = state_indices; R.o = o;
    R.cu = P.varlen ? p->cu_seqlens_dev : nullptr;
    R.N = (int)P.N;
    R.H = (int)p->heads;
    R.dense_T = P.varlen ? 0 : (int)p->seqlen;
    R.tokens = P.tokens;
    R.num_slots = num_slots;
    R.scale = p->scale;
    R.norm = p->qk_l2norm;
    R.ldq = ldq;
    R.ldv = ldv;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t err = timed("recurrent", s, [&] { return gdn::launch_recurrent(R, (int)p->dk, (int)p->dv, P.bf16, s); });
    if (err != hipSuccess) return hip_fail(err, "recurrent forward launch");
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "unexpected exception in gdn_recurrent_fwd");
  }
}

int gdn_profile_events(void* const* events, int n_pairs) {
  if (events && n_pairs > 0) {
    g_prof.events = events;
    g_prof.pairs = n_pairs;
    g_prof.count = 0;
  } else {
    // stop bracketing; the record of the last run stays readable
    g_prof.events = nullptr;
    g_prof.pairs = 0;
  }
  return 0;
}

int gdn_profile_count(void) { return g_prof.count; }

const char* gdn_profile_name(int i) {
  if (i < 0 || i >= g_prof.count || i >= 512 || !g_prof.names[i]) return "";
  return g_prof.names[i];
}

size_t gdn_fwd_workspace_bytes(const gdn_problem* p) {
  try {
    Layout L;
    return plan_problem(p, &L) == GDN_OK ? L.fwd_bytes : 0;
  } catch (...) {
    return 0;
  }
}

size_t gdn_bwd_workspace_bytes(const gdn_problem* p) {
  try {
    Layout L;
    if (plan_problem(p, &L) != GDN_OK) return 0;
    return L.bwd_bytes;
  } catch (...) {
    return 0;
  }
}

gdn_status gdn_fwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const float* h0, void* o, float* ht, void* workspace,
                   size_t workspace_bytes, void* stream) {
  try {
    Layout L;
    gdn_status st = plan_problem(p, &L);
    if (st != GDN_OK) return st;
    st = check_fwd_args(L, q, k, v, g, beta, h0, o, ht, workspace, true);
    if (st != GDN_OK) return st;
    if (workspace && ((uintptr_t)workspace) % ALIGN)
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < L.fwd_bytes)
      return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, L.fwd_bytes);
    return fwd_launch(p, L, q, k, v, g, beta, h0, o, ht, reinterpret_cast<char*>(workspace),
                      reinterpret_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(GDN_ERR_HIP, "unexpected exception in gdn_fwd");
  }
}

gdn_status gdn_fwd_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* h0, void* o, float* ht,
                           void* stream) {
  try {
    Layout L;
    gdn_status st = plan_problem(p, &L);
    if (st != GDN_OK) return st;
    st = check_fwd_args(L, q, k, v, g, beta, h0, o, ht, nullptr, false);
    if (st != GDN_OK) return st;
    if (L.fwd_bytes > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
      return fail(GDN_ERR_UNSUPPORTED,
                  "gdn_fwd_noalloc: the problem needs %zu bytes of scratch, more than the library's static "
                  "%zu bytes (use gdn_fwd with a workspace)",
                  L.fwd_bytes, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int dev = 0;
    hipError_t e = stream_device(s, &dev);
    if (e != hipSuccess) return hip_fail(e, "gdn_fwd_noalloc: device of the stream");
    char* ws = nullptr;
    if ((e = static_scratch(dev, &ws)) != hipSuccess) return hip_fail(e, "gdn_fwd_noalloc: static scratch address");
    return fwd_launch(p, L, q, k, v, g, beta, h0, o, ht, ws, s);
  } catch (...) {
    return fail(GDN_ERR_HIP, "unexpected exception in gdn_fwd_noalloc");
  }
}

gdn_status gdn_bwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const float* h0, const void* d_o, const float* dht, void* dq,
                   void* dk, void* dv, float* dg, float* dbeta, float* dh0, const void* fwd_workspace,
                   void* workspace, size_t workspace_bytes, void* stream) {
  try {
    Layout L;
    gdn_status st = plan_problem(p, &L);
    if (st != GDN_OK) return st;
    const size_t ob = (size_t)(L.tokens * L.H * L.DV) * L.esz;
    const size_t gb = (size_t)(L.tokens * L.H) * sizeof(float);
    const size_t sb = (size_t)(L.N * L.H * L.DK * L.DV) * sizeof(float);
    auto sq_ = [&](const void* x, const char* nm) { return strided(x, L.tokens, L.H * L.DK, L.ldq, L.esz, nm); };
    auto sv_ = [&](const void* x, const char* nm) { return strided(x, L.tokens, L.H * L.DV, L.ldv, L.esz, nm); };
    const Range rq = sq_(q, "q"), rk = sq_(k, "k"), rv = sv_(v, "v"), rdq = sq_(dq, "dq"), rdk = sq_(dk, "dk"),
                rdv = sv_(dv, "dv");
    const Range req[] = {rq, rk, rv, {g, gb, "g"}, {beta, gb, "beta"},
                         {d_o, ob, "do"}, rdq, rdk, rdv, {dg, gb, "dg"},
                         {dbeta, gb, "dbeta"}, {workspace, L.bwd_bytes, "workspace"}};
    const Range opt[] = {{h0, sb, "h0"}, {dht, sb, "dht"}, {dh0, sb, "dh0"},
                         {fwd_workspace, L.fwd_bytes, "fwd_workspace"}};
    const Range outs[] = {rdq, rdk, rdv, {dg, gb, "dg"}, {dbeta, gb, "dbeta"},
                          {dh0, sb, "dh0"}, {workspace, L.bwd_bytes, "workspace"}};
    const Range ins[] = {rq, rk, rv, {g, gb, "g"}, {beta, gb, "beta"},
                         {h0, sb, "h0"}, {d_o, ob, "do"}, {dht, sb, "dht"},
                         {fwd_workspace, L.fwd_bytes, "fwd_workspace"}};
    st = check_ptrs(req, 12, opt, 4, outs, 7, ins, 9);
    if (st != GDN_OK) return st;
    if (workspace && ((uintptr_t)workspace) % ALIGN)
      return fail(GDN_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (fwd_workspace && ((uintptr_t)fwd_workspace) % ALIGN)
      return fail(GDN_ERR_INVALID_ARGUMENT, "fwd_workspace is not 256-byte aligned");
    if (workspace_bytes < L.bwd_bytes)
      return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, L.bwd_bytes);

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = reinterpret_cast<char*>(workspace);
    // forward context: from the caller's forward workspace, or recomputed here
    char* ctx = fwd_workspace ? const_cast<char*>(reinterpret_cast<const char*>(fwd_workspace)) : ws;
    gdn::Params P = base_params(p, L, ctx, s);
    P.q = q; P.k = k; P.v = v; P.g = g; P.beta = beta; P.h0 = h0;
    P.dO = d_o; P.dht = dht; P.dq = dq; P.dk = dk; P.dv = dv; P.dg = dg; P.dbeta = dbeta; P.dh0 = dh0;
    P.Z = ws + L.Z; P.WnT = ws + L.WnT; P.Ktn = ws + L.Ktn;
    P.HPf = ws + L.HPf; P.dVf = ws + L.dVf; P.dVl = ws + L.dVl;
    if (L.l2norm) P.qinv = reinterpret_cast<float*>(ws + L.qinv);
    const int D = (int)L.D;
    hipError_t e;
    if (!fwd_workspace) {
      if (L.varlen && (e = timed("plan", s, [&] { return gdn::launch_plan(P, s); })) != hipSuccess) return hip_fail(e, "plan launch");
      if ((e = timed("fwd_prep", s, [&] { return gdn::launch_fwd_prep(P, D, L.bf16, s); })) != hipSuccess) return hip_fail(e, "fwd_prep launch");
      if ((e = timed("fwd_state", s, [&] { return gdn::launch_fwd_state(P, D, L.bf16, false, s); })) != hipSuccess) return hip_fail(e, "fwd_state launch");
    }
    if ((e = timed("bwd_prep", s, [&] { return gdn::launch_bwd_prep(P, D, L.bf16, s); })) != hipSuccess) return hip_fail(e, "bwd_prep launch");
    if ((e = timed("bwd_state", s, [&] { return gdn::launch_bwd_state(P, D, L.bf16, s); })) != hipSuccess) return hip_fail(e, "bwd_state launch");
    if ((e = timed("bwd_grad", s, [&] { return gdn::launch_bwd_grad(P, D, L.bf16, s); })) != hipSuccess) return hip_fail(e, "bwd_grad launch");
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "unexpected exception in gdn_bwd");
  }
}

}  // extern "C"
