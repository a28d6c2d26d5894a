/*
 * gdn.h -- C ABI of libgdn.so: the Gated DeltaNet (GDN) chunked gated
 * delta-rule operator, forward and backward, on one AMD MI355X (gfx950).
 *
 * The operator is the linear-attention core of Qwen3.5 that the XTuner /
 * Ascend 910C training article rebuilds natively (section 3.1.2, "GDN linear
 * attention rebuilt natively in Ascend C"; Fig. 7 lists its kernel family:
 * the forward state update that also runs inside the backward, the reverse
 * pass through the state-transition chain, the local dv update and the
 * dq/dk/dw/dg projection; Fig. 8 adds the triangular-solve helper).  The
 * article prints no formula; the recurrence implemented is the gated delta
 * rule, per sequence and head:
 *
 *     S_t = exp(g_t) * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * S_t is d_v x d_k.  It crosses this interface transposed: a state tensor is
 * [N][H][d_k][d_v] fp32 with element (n, h, i, j) = S[j][i] of sequence n,
 * head h.
 *
 * Layouts (contiguous, last index fastest; B*T tokens in total):
 *   q, k, dq, dk : [B][T][H][d_k]      dtype of the problem (fp32 or bf16)
 *   v, o, do, dv : [B][T][H][d_v]      dtype of the problem
 *   g, beta, dg, dbeta : [B][T][H]     fp32 (g is the natural-log decay)
 *   h0, ht, dht, dh0   : [N][H][d_k][d_v] fp32
 * With qkv_token_stride = s > 0, q, k, v, dq, dk, dv instead advance by s
 * elements per token ([B*T][s] buffers in which each occupies H*d columns);
 * o and do stay as above.  Interleaved outputs dq, dk, dv are allowed as long
 * as no element is shared.
 * Dense problems have N = B sequences of T tokens each.  Packed
 * variable-length problems have B = 1, T = total tokens and N sequences
 * given by cu_seqlens (int32, N+1 entries, cu[0] = 0, non-decreasing,
 * cu[N] = T; zero-length sequences are allowed and pass their state through).
 * The host copy of cu_seqlens is validated and sizes the launches; the device
 * copy, which the kernels read, must hold the same values.  If it does not,
 * the results are unspecified, but the kernels clamp what they take from it
 * so that no read or write leaves the buffers the host copy describes.
 *
 * Ownership and execution:
 *  - The caller owns every buffer.  The library never allocates, frees or
 *    synchronises device memory and is reentrant; its only state is
 *    thread-local (the last error message and the timing diagnostics below),
 *    apart from the static scratch array of gdn_fwd_noalloc (one per GPU, see
 *    there).
 *  - All device work is enqueued on the caller's stream (hipStream_t passed
 *    as void*, NULL = the null stream); the calls return without waiting.
 *  - Inputs are read-only.  Outputs are fully overwritten (never
 *    accumulated) and must not alias any input, each other or the workspace.
 *  - The workspace is caller-provided device memory of at least the size
 *    the *_workspace_bytes query returns, 256-byte aligned.  It is
 *    stream-ordered scratch: reusable once the stream has passed the call.
 *  - Every device pointer must be 16-byte aligned.
 *
 * Errors: every argument is checked on the host before any HIP call; a
 * failing check returns GDN_ERR_INVALID_ARGUMENT, GDN_ERR_UNSUPPORTED or
 * GDN_ERR_WORKSPACE_TOO_SMALL and enqueues nothing.  A launch failure returns
 * GDN_ERR_HIP.  Device faults surface at the caller's next synchronisation.
 * gdn_last_error_message() returns a thread-local description of the last
 * non-OK return.  Nothing aborts, prints or throws across this interface.
 *
 * Supported set (gdn_fwd, gdn_bwd): d_k and d_v each in {64, 128} (equal or
 * not), chunk = 64, dtype fp32 or bf16 (forward and backward in each), any
 * T >= 0 (a problem with no tokens enqueues only state copies).  Anything else
 * returns GDN_ERR_UNSUPPORTED.
 *
 * In-operator L2 normalisation (qk_l2norm = 1) is the usual prologue of the
 * GDN layer (Qwen3.5 normalises q and k per head before the recurrence).
 * The norms are taken inside the kernels that read the rows; the forward
 * keeps the reciprocal key norms in its workspace with the rest of the
 * forward context, and gdn_bwd reads them from there (or recomputes them).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 7

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1,
  GDN_ERR_UNSUPPORTED = 2,
  GDN_ERR_WORKSPACE_TOO_SMALL = 3,
  GDN_ERR_HIP = 4
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef struct {
  int64_t batch;   /* B; must be 1 when cu_seqlens are given                    */
  int64_t seqlen;  /* T: tokens per batch row, or total packed tokens (varlen)  */
  int64_t heads;   /* H                                                          */
  int64_t dk;      /* key/query head dim                                         */
  int64_t dv;      /* value head dim (64 or 128; may differ from dk)             */
  int64_t chunk;   /* chunk length of the chunked form; must be 64               */
  int64_t num_seqs;                /* N when varlen; ignored when dense            */
  const int32_t* cu_seqlens_host;  /* [N+1] host copy: validation and launch sizes */
  const int32_t* cu_seqlens_dev;   /* [N+1] device copy read by the kernels        */
                                   /* both NULL: dense; both non-NULL: varlen      */
  float scale;     /* o = scale * S q                                             */
  gdn_dtype dtype; /* dtype of q, k, v, o, do, dq, dk, dv                         */
  int32_t qk_l2norm;  /* 0: q and k are used as given.  1: every (token, head) row */
                      /* of q and of k is divided by max(||row||_2, 1e-12) inside  */
                      /* the operator (rounded to the problem dtype), and dq, dk   */
                      /* are the gradients with respect to the raw rows.           */
  int32_t qkv_token_stride;  /* 0: q, k, dq, dk hold H*dk and v, dv H*dv elements  */
                             /* per token (contiguous).  > 0: all six advance by   */
                             /* this many elements per token (slices of one        */
                             /* [tokens][stride] buffer such as a conv1d output);  */
                             /* >= H*max(dk, dv), a multiple of 8 (bf16) or 4      */
                             /* (fp32); o and do stay contiguous                   */
} gdn_problem;

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

/* Workspace sizes in bytes for a valid problem; 0 if the problem is invalid
 * or unsupported (the matching call then reports why). */
size_t gdn_fwd_workspace_bytes(const gdn_problem* p);
size_t gdn_bwd_workspace_bytes(const gdn_problem* p);

/* Forward: o and (if ht != NULL) the final states.
 *   q, k, v : device, layouts above, problem dtype
 *   g, beta : device fp32 [B][T][H]
 *   h0      : device fp32 [N][H][dk][dv] initial states, or NULL for zeros
 *   o       : device output, problem dtype
 *   ht      : device fp32 [N][H][dk][dv] final states, or NULL to skip
 *   workspace / workspace_bytes : device scratch, >= gdn_fwd_workspace_bytes
 * On return the workspace also holds the per-chunk forward context
 * (decays, WY factors, chunk-entry states, corrected values); gdn_bwd may
 * reuse it (see fwd_workspace below) as long as it is left untouched. */
gdn_status gdn_fwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* h0, void* o, float* ht,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Backward of L = sum_t <do_t, o_t> + <dht, ht>:
 *   do      : device upstream gradient of o, problem dtype
 *   dht     : device fp32 gradient of the final states, or NULL for zero
 *   dq, dk, dv : device outputs, problem dtype
 *   dg, dbeta  : device fp32 outputs [B][T][H]
 *   dh0     : device fp32 [N][H][dk][dv] gradient of h0, or NULL to skip
 *             (defined also when h0 is NULL: the gradient at a zero state)
 *   fwd_workspace : NULL, or the workspace of a completed gdn_fwd call with
 *             the same problem and the same q, k, v, g, beta, h0, left
 *             untouched since; then the forward context is read from it
 *             instead of being recomputed.  Anything else there gives
 *             undefined results.
 *   workspace / workspace_bytes : device scratch, >= gdn_bwd_workspace_bytes
 */
gdn_status gdn_bwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* h0, const void* d_o,
                   const float* dht, void* dq, void* dk, void* dv, float* dg, float* dbeta,
                   float* dh0, const void* fwd_workspace, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ---- Allocation-free forward ---------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * computation and kernels as gdn_fwd (bitwise the same o and ht), with the
 * workspace taken from a static device array inside the library instead of
 * from the caller: GDN_NOALLOC_SCRATCH_BYTES (128 MiB), one copy on every GPU
 * the library runs on, held until the process ends.  The call allocates
 * nothing; the first call on a GPU looks up that GPU's copy.
 *   - A problem whose gdn_fwd_workspace_bytes exceeds the limit returns
 *     GDN_ERR_UNSUPPORTED before any HIP call (at d = 128 in bf16 the limit
 *     holds about 1,150 (64-token chunk, head) pairs, e.g. T = 4096, H = 16).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero).  Calls that
 *     overlap in time on one GPU (other streams, other threads) race; the
 *     caller must order them.  For the same reason the forward context left in
 *     the array is not for gdn_bwd: pass gdn_fwd's own workspace there.
 * Arguments, layouts, streams and errors as for gdn_fwd. */
#define GDN_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
gdn_status gdn_fwd_noalloc(const gdn_problem* p, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const float* h0, void* o, float* ht,
                           void* stream);

/* ---- Recurrent (decoding) forward ----------------------------------------
 * The same recurrence as gdn_fwd, taken token by token for the decoding
 * regime: each sequence brings a few new tokens and its state is read and
 * written once, in place.  (The article covers training only; the operator
 * is the one of its §3.1.2.)  For each sequence and head, token by token:
 *     S <- exp(g) S (I - beta k k^T) + beta v k^T,   o = scale S q
 * with q, k L2-normalised first when qk_l2norm = 1, in fp32.
 *
 * The problem is a gdn_problem with these differences: dk and dv may differ
 * (each in {64, 128}); `chunk` is ignored; seqlen is the number of new tokens
 * per sequence (dense) or their packed total (cu_seqlens).  Layouts of q, k,
 * v, g, beta and o as for gdn_fwd.
 *   state          : device fp32 [num_slots][H][dk][dv] holding S^T, read and
 *                    overwritten in place
 *   state_indices  : NULL (sequence n uses slot n; num_slots >= N), or device
 *                    int32 [N]: sequence n uses slot state_indices[n].  An
 *                    index outside [0, num_slots) skips the sequence: its o
 *                    rows are written as zeros and no state is touched.  Two
 *                    sequences must not name the same slot.
 * Ownership, streams and errors as for gdn_fwd; o must not overlap the
 * inputs or the state.  Any number of tokens per sequence is allowed; the
 * tokens of one sequence run one after another, so long prompts belong to
 * gdn_fwd (which leaves the final state in ht for a following decode). */
gdn_status gdn_recurrent_fwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, float* state,
                             const int32_t* state_indices, int64_t num_slots, void* o,
                             void* stream);

/* ---- Gated RMSNorm on the operator's output ------------------------------
 * The output gate of the GDN layer, as the XTuner / Ascend 910C Qwen3.5
 * training article takes it apart in §2.4 (Fig. 3C: squares, mean, eps,
 * reciprocal square root, the products with the row and the weight, the
 * gate's SiLU and its product) and fuses it in §3.1.2 (Fig. 6: one forward
 * and one backward kernel).  For every row x of `dim` values (one token and
 * head of the operator's output o), gate row z and weight w[dim]:
 *     y = x * (mean(x^2) + eps)^(-1/2) * w * z * sigmoid(z)
 * computed in fp32 and rounded once to the problem dtype.  The backward
 * returns dx, dz (problem dtype) and dw = the sum over all rows (fp32).
 *
 * Layouts: x, z, y, dy, dx, dz are [rows][dim] row-major and contiguous (a
 * [B][T][H][dv] tensor is rows = B*T*H rows of dim = dv); w and dw are fp32
 * [dim].  Device pointers, 16-byte aligned; the workspace 256-byte aligned.
 * Ownership, streams and errors as for gdn_fwd: every buffer is the caller's,
 * nothing is allocated or synchronised, all work is enqueued on `stream`,
 * every argument is checked before any HIP call.  Outputs are overwritten
 * and must not overlap the inputs or each other.  With eps = 0 a zero row
 * gives NaN (0 * inf), as the formula does.  Supported set: dim in {64, 128},
 * dtype fp32 or bf16, rows >= 0 (rows = 0: the backward writes dw = 0).
 * Results are bitwise reproducible for a given problem. */
typedef struct {
  int64_t rows;     /* number of rows (tokens x heads), >= 0                    */
  int64_t dim;      /* values per row                                           */
  float eps;        /* added to the mean square: finite, >= 0                   */
  gdn_dtype dtype;  /* dtype of x, z, y, dy, dx, dz                             */
} gdn_gated_norm_problem;

/* Workspace of gdn_gated_rmsnorm_bwd in bytes (per-workgroup partial sums of
 * dw, at most 512 KiB); 0 if the problem is invalid or unsupported. */
size_t gdn_gated_rmsnorm_bwd_workspace_bytes(const gdn_gated_norm_problem* p);

/* Forward: y from x, z and w. */
gdn_status gdn_gated_rmsnorm_fwd(const gdn_gated_norm_problem* p, const void* x, const void* z,
                                 const float* w, void* y, void* stream);

/* Backward of L = sum(dy * y): dx, dz and dw (all three written). */
gdn_status gdn_gated_rmsnorm_bwd(const gdn_gated_norm_problem* p, const void* x, const void* z,
                                 const float* w, const void* dy, void* dx, void* dz, float* dw,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* ---- Causal depthwise conv1d over packed sequences -----------------------
 * The GDN layer's short causal convolution, which the XTuner / Ascend 910C
 * Qwen3.5 training article (§3.1.2, Fig. 8) moves from a loop of slices and
 * pads per sequence into one native forward and one backward kernel.  For
 * channel c, kernel size K and token t of a sequence whose first token is t0:
 *     pre = bias[c] + sum_{j<K} w[c][j] * x[t - (K-1) + j][c]  (x = 0 before t0)
 *     y   = pre * sigmoid(pre) with the activation, pre without it
 * in fp32, rounded once.  Nothing crosses a sequence start.  The backward
 * returns dx (same sequence only), dw = sum_t dpre[t] x[t - (K-1) + j] and,
 * if dbias != NULL, dbias = sum_t dpre[t] (fp32, over all tokens).
 *
 * Layouts: x, y, dy, dx are [B*T][channels] row-major (channels last; for
 * packed input B = 1 and cu_seqlens as in gdn_problem); w is fp32
 * [channels][K] (a depthwise conv1d weight [C][1][K]); bias and dbias are fp32
 * [channels] or NULL.  Device pointers 16-byte aligned, the workspace 256-byte
 * aligned.  Ownership, streams, errors and non-overlap of outputs as for
 * gdn_fwd.  Supported set: K in [1, 4], channels a positive multiple of 4,
 * dtype fp32 or bf16, any T >= 0.  Results are bitwise reproducible. */
typedef struct {
  int64_t batch;       /* B; must be 1 when cu_seqlens are given                     */
  int64_t seqlen;      /* T: tokens per batch row, or total packed tokens            */
  int64_t channels;    /* C                                                          */
  int64_t kernel_size; /* K                                                          */
  int64_t num_seqs;                /* N when packed; ignored when dense              */
  const int32_t* cu_seqlens_host;  /* [N+1] host copy (validation), or NULL          */
  const int32_t* cu_seqlens_dev;   /* [N+1] device copy read by the kernels, or NULL */
  int32_t activation;  /* 0: none, 1: SiLU                                           */
  gdn_dtype dtype;     /* dtype of x, y, dy, dx                                      */
} gdn_conv_problem;

/* Workspace of gdn_causal_conv1d_bwd in bytes (per-grid-row partial sums of
 * dw and dbias: at most 64 * channels * (K+1) fp32); 0 if the problem is
 * invalid or unsupported. */
size_t gdn_causal_conv1d_bwd_workspace_bytes(const gdn_conv_problem* p);

/* Forward: y from x, w and bias (NULL: no bias). */
gdn_status gdn_causal_conv1d_fwd(const gdn_conv_problem* p, const void* x, const float* w,
                                 const float* bias, void* y, void* stream);

/* Backward of L = sum(dy * y): dx, dw and (if dbias != NULL) dbias. */
gdn_status gdn_causal_conv1d_bwd(const gdn_conv_problem* p, const void* x, const float* w,
                                 const float* bias, const void* dy, void* dx, float* dw,
                                 float* dbias, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* ---- Timing diagnostics ------------------------------------------------
 * gdn_profile_events: bracket each kernel launched by the following
 * gdn_fwd / gdn_bwd / gdn_recurrent_fwd / gdn_gated_rmsnorm_* / gdn_causal_conv1d_* calls made on
 * this thread with caller-created HIP events
 * (hipEvent_t passed as void*): events[2i] is recorded on the call's stream
 * just before launch i and events[2i+1] just after it, for the first n_pairs
 * launches; later launches run unbracketed.  Enabling restarts the launch
 * count.  events == NULL or n_pairs <= 0 turns bracketing off and leaves the
 * record of the last run readable.  The events stay owned by the caller.
 * The state is thread-local and holds no device memory.  Returns 0.
 * gdn_profile_count: launches bracketed since bracketing was last enabled.
 * gdn_profile_name: static kernel name of bracketed launch i ("" if none). */
int gdn_profile_events(void* const* events, int n_pairs);
int gdn_profile_count(void);
const char* gdn_profile_name(int i);

/* Static name of a status code. */
const char* gdn_status_string(gdn_status s);

/* Thread-local description of the last non-OK status returned on this
 * thread ("" if none). */
const char* gdn_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
