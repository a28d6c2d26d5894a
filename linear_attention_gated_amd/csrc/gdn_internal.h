// gdn_internal.h -- parameters and workspace layout shared by the host
// planner (api.cpp) and the kernels (*.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int CHUNK = 64;   // chunk length of the chunked form
constexpr int REC = 512;    // elements per fragment record (64 lanes x 8)
constexpr int AREC = 256;   // elements per accumulator record (64 lanes x 4)

// Record counts per (chunk, head), for head dim D = max(dk, dv):
//   Wn  F(-W; r, i)      [4][D/32]        forward WY factor, negated
//   Ktf F(Kt; i, s)      [D/16][2]        decayed keys, transposed
//   Ua  acc U[r][j]      [D/16][4]        WY values (accumulator records)
//   Hf  F(h; j, i)       [D/16][D/32]     chunk-entry state
//   Vf  F(V'; j, s)      [D/16][2]        corrected values
//   Tm  T[r][s] fp32     64 x 64 row-major  (I + A)^-1, upper blocks zero
// and, with in-operator normalisation, per (token, head) fp32 (negative:
// the row's norm is below the floor and the value is -1 / floor):
//   kinv                 1 / max(||k||_2, 1e-12), written by the WY prep
//   qinv                 1 / max(||q||_2, 1e-12), backward workspace, written
//                        by the backward prep (the forward output pass
//                        computes its own, with the same arithmetic)
//   Z   acc Z[i][j]      [D/16 jb][D/16 ib]  backward: (scale Gam Q)^T dO
//   WnT F(-W; i, r)      [D/16][2]        backward: WY factor, transposed
//   Ktn F(Kt; s, i)      [4][D/32]        backward: decayed keys
//   dVl acc dV'loc[s][j] [D/16][4]        backward: intra-chunk part of dV'
//   HPf F(H'; j, i)      [D/16][D/32]     backward: state gradient after the chunk
//   dVf F(dV'; j, r)     [D/16][2]        backward: gradient of V'
struct Params {
  int H, N, NC;           // heads, sequences, chunks
  float scale;
  int dense_T;            // tokens per sequence when dense (cu == nullptr)
  int total_tokens;       // B * T
  const int32_t* cu;      // device cu_seqlens or nullptr

  const void *q, *k, *v;
  const float *g, *beta, *h0;
  const void* dO;
  const float* dht;

  void* o;
  float* ht;
  void *dq, *dk, *dv;
  float *dg, *dbeta, *dh0;

  int4* chunk_tab;        // per chunk: first token, length, sequence, index in sequence
  int4* seq_tab;          // per sequence: first chunk, chunk count, first token, length

  float* gamma;           // [NC][H][64] chunk-local cumulative log decay
  void *Wn, *Ktf, *Ua, *Hf, *Vf;
  float* Tm;
  int qk_l2norm;          // 1: q and k rows L2-normalised inside the operator
  // Head dims.  The kernels run at D = max(dk, dv); a narrower q/k (dk < D)
  // or v (dv < D) is read with zeros past its width and its outputs are
  // written only up to it: zero columns stay zero through every product, so
  // the padded problem has exactly the rectangular one's results.
  int kdim, vdim;
  long long ldq, ldv;     // token strides (elements) of q, k, dq, dk and of v, dv
  float* kinv;            // reciprocal key norms [tokens][H] (forward context), sign-encoded
  float* qinv;            // reciprocal query norms [tokens][H] (backward workspace)
  void *WnT, *Ktn, *HPf, *dVf;
  void *Z, *dVl;
  int dma_rot;             // 1: the column-block workgroups of a state pass start their shared reads at different pieces
  int state_cpw;           // 16-column blocks of d_v per state-pass workgroup: 1 or 2 (2 implies dma_rot)
  int grad_ahead;          // k_bwd_grad: workgroups one round holds (a multiple of 8), the prefetch distance
};

// Chunk c: (first token, length, sequence, index in sequence).  Dense
// problems (no cu_seqlens) are arithmetic; packed problems read the table
// the planner built.
__device__ __forceinline__ int4 chunk_info(const Params& p, int c) {
  if (p.cu) return p.chunk_tab[c];
  const int ncs = (p.dense_T + 63) / 64;
  const int n = c / ncs, j = c - n * ncs;
  return make_int4(n * p.dense_T + 64 * j, min(64, p.dense_T - 64 * j), n, j);
}
// Sequence n: (first chunk, chunk count, first token, length).
__device__ __forceinline__ int4 seq_info(const Params& p, int n) {
  if (p.cu) return p.seq_tab[n];
  const int ncs = (p.dense_T + 63) / 64;
  return make_int4(n * ncs, ncs, n * p.dense_T, p.dense_T);
}

// Launchers (each returns the first launch error, hipSuccess otherwise).
hipError_t launch_plan(const Params& p, hipStream_t s);
hipError_t launch_fwd_prep(const Params& p, int D, bool bf16, hipStream_t s);
hipError_t launch_fwd_state(const Params& p, int D, bool bf16, bool write_ht, hipStream_t s);
hipError_t launch_fwd_out(const Params& p, int D, bool bf16, hipStream_t s);
hipError_t launch_bwd_prep(const Params& p, int D, bool bf16, hipStream_t s);
hipError_t launch_bwd_state(const Params& p, int D, bool bf16, hipStream_t s);
hipError_t launch_bwd_grad(const Params& p, int D, bool bf16, hipStream_t s);

// Gated RMSNorm on the operator's output (gnorm.hip): rows of D values,
// row-major and contiguous.
struct GnormParams {
  const void *x, *z, *dy;   // [rows][D], problem dtype
  const float* w;           // [D]
  void *y, *dx, *dz;        // [rows][D], problem dtype
  float* dw;                // [D]
  float* part;              // [D][nblk] per-workgroup partials of dw (workspace)
  long long rows;
  float eps;
  int nblk;                 // set by the launcher
};
constexpr int GNORM_MAX_BWD_BLOCKS = 1024;
// Workgroups of the forward (bwd = false) or backward kernel for `rows` rows.
int gnorm_blocks(long long rows, int D, bool bf16, bool bwd);
hipError_t launch_gnorm_fwd(const GnormParams& p, int D, bool bf16, hipStream_t s);
// backward kernel (dx, dz, per-workgroup dw partials), then the fixed-order
// sum of the partials
hipError_t launch_gnorm_bwd(const GnormParams& p, int D, bool bf16, hipStream_t s);
hipError_t launch_gnorm_dw(const GnormParams& p, int D, bool bf16, hipStream_t s);

// Causal depthwise conv1d over packed sequences (conv.hip): x, y, dy, dx are
// [tokens][C], w [C][K], bias [C], fp32 parameters.
struct ConvParams {
  const void *x, *dy;
  const float *w, *bias;    // bias may be nullptr
  void *y, *dx;
  float *dw, *dbias;        // dbias may be nullptr
  float* part;              // [ntiles][C][K+1] per-workgroup-row partials (workspace)
  const int32_t* cu;        // device cu_seqlens, or nullptr (dense)
  int N;                    // sequences
  int dense_T;              // tokens per sequence when dense
  long long tokens;
  int C, K, act, ntiles;    // ntiles: set by the launchers
};
constexpr int CONV_MAX_BWD_ROWS = 64;
// rows of the backward grid (and of its partials) for `tokens` tokens of C channels
int conv_bwd_rows(long long tokens, int C);
hipError_t launch_conv_fwd(const ConvParams& p, bool bf16, hipStream_t s);
hipError_t launch_conv_bwd(const ConvParams& p, bool bf16, hipStream_t s);
hipError_t launch_conv_dw(const ConvParams& p, hipStream_t s);

// Recurrent (decoding) forward (recur.hip): the state [num_slots][H][dk][dv]
// fp32 updated in place; sequence n uses slot idx[n] (or n when idx is null).
struct RecParams {
  const void *q, *k, *v;    // [tokens][H][dk], [tokens][H][dk], [tokens][H][dv]
  const float *g, *beta;    // [tokens][H]
  float* state;
  const int32_t* idx;       // device [N] or nullptr
  void* o;                  // [tokens][H][dv]
  const int32_t* cu;        // device cu_seqlens or nullptr (dense)
  int N, H, dense_T;
  long long tokens;         // B * T: cu values are clamped to [0, tokens]
  long long num_slots;
  float scale;
  int norm;                 // 1: q and k rows L2-normalised
  long long ldq, ldv;       // token strides (elements) of q, k and of v
};
hipError_t launch_recurrent(const RecParams& p, int dk, int dv, bool bf16, hipStream_t s);

// Grid of the sequential kernels: one wave per (sequence, head, 16-column
// block), padded so that the column blocks of one (sequence, head) share an
// XCD (workgroup ids are dealt round-robin over the 8 XCDs).
inline int state_grid(int units, int D, int cpw = 1) {
  const int nj = D / 16 / cpw;   // workgroups per (sequence, head): cpw column blocks each
  const int groups = (units + 7) / 8;
  return groups * 8 * nj;
}

}  // namespace gdn
