// gnorm.hip -- gated RMSNorm on the operator's output, forward and backward.
//
// XTuner / Ascend 910C Qwen3.5 training article, §2.4 (Fig. 3C: the output
// gate's RMSNorm taken apart into squares, mean, eps, reciprocal root, the
// products with the row and the weight, the gate's SiLU and its product) and
// §3.1.2 (Fig. 6: the same chain as one forward and one backward kernel).
// Per row x (one token and head, D values), gate row z and weight w[D]:
//     r = (mean x^2 + eps)^(-1/2),  n = r x,  a = n w,  y = a silu(z)
// and, for an upstream dy,
//     da = dy silu(z),  dz = dy a sigmoid(z) (1 + z (1 - sigmoid(z))),
//     dn = da w,  dx = r (dn - n mean(dn n)),  dw = sum over rows of da n.
// All arithmetic is fp32 (the reciprocal root and the sigmoid's reciprocal
// are the hardware's 1-ulp instructions); every output is rounded once.
//
// HBM-bound: each value is read and written once.  A row is D * sizeof(E)
// bytes in LPR 16-byte pieces held by LPR consecutive lanes, so its sums are
// a butterfly over LPR lanes (bitwise the same in every lane).  Thread t of
// a grid of S threads takes pieces t, t + S, t + 2S, ... (S is a multiple of
// LPR, so all of a thread's pieces lie in one column block), PPT of them per
// round with every read issued before any arithmetic.  dw is reduced in a
// fixed order: per workgroup over its threads, then over the workgroups in
// a second kernel (one wave per column, a fixed butterfly), so results are
// bitwise reproducible.
#include <hip/hip_runtime.h>

#include "frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int NT = 256;   // threads per workgroup
constexpr int PPT = 2;    // pieces per thread per round

template <typename E> struct PieceT;
template <> struct PieceT<bf16> {
  static constexpr int N = 8;
  using F = f32x8;
  static __device__ __forceinline__ F to_f(i32x4 v) { return __builtin_convertvector(__builtin_bit_cast(bf16x8, v), f32x8); }
  static __device__ __forceinline__ i32x4 from_f(F f) { return __builtin_bit_cast(i32x4, __builtin_convertvector(f, bf16x8)); }
};
template <> struct PieceT<float> {
  static constexpr int N = 4;
  using F = f32x4;
  static __device__ __forceinline__ F to_f(i32x4 v) { return __builtin_bit_cast(f32x4, v); }
  static __device__ __forceinline__ i32x4 from_f(F f) { return __builtin_bit_cast(i32x4, f); }
};

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// 1 / (1 + e^-z) with the hardware reciprocal (1 ulp); saturates to 0 and 1
__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

template <typename E, int D>
struct GnGeom {
  static constexpr int EPP = PieceT<E>::N;    // values per piece
  static constexpr int LPR = D / EPP;         // lanes (pieces) per row
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0 && NT % LPR == 0, "a row must sit in one wave");
};

template <typename E, int D>
__global__ __launch_bounds__(NT) void k_gnorm_fwd(GnormParams p) {
  using P = PieceT<E>;
  using G = GnGeom<E, D>;
  constexpr int EPP = G::EPP, LPR = G::LPR;
  const long long npieces = p.rows * LPR;
  const long long S = (long long)gridDim.x * NT;
  const int c = threadIdx.x % LPR;   // column block of every piece of this thread
  float wv[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) wv[e] = p.w[c * EPP + e];
  const i32x4* X = reinterpret_cast<const i32x4*>(p.x);
  const i32x4* Z = reinterpret_cast<const i32x4*>(p.z);
  i32x4* Y = reinterpret_cast<i32x4*>(p.y);
  const float inv_d = 1.f / (float)D;
  for (long long q0 = (long long)blockIdx.x * NT + threadIdx.x; q0 < npieces; q0 += PPT * S) {
    i32x4 xv[PPT], zv[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {   // unconditional reads (piece 0 out of range): all in flight
      const long long q = q0 + k * S, qc = q < npieces ? q : 0;
      xv[k] = X[qc];
      zv[k] = Z[qc];
    }
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const long long q = q0 + k * S;
      const typename P::F xf = P::to_f(xv[k]), zf = P::to_f(zv[k]);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) ss += xf[e] * xf[e];
      ss = row_sum<LPR>(ss);   // the whole row group is in range or out of it together
      const float r = rsqrtf(ss * inv_d + p.eps);
      typename P::F yf;
#pragma unroll
      for (int e = 0; e < EPP; ++e) yf[e] = (xf[e] * r * wv[e]) * (zf[e] * sigmoid(zf[e]));
      if (q < npieces) Y[q] = P::from_f(yf);
    }
  }
}

template <typename E, int D>
__global__ __launch_bounds__(NT) void k_gnorm_bwd(GnormParams p) {
  using P = PieceT<E>;
  using G = GnGeom<E, D>;
  constexpr int EPP = G::EPP, LPR = G::LPR;
  __shared__ float red[NT * EPP];
  const long long npieces = p.rows * LPR;
  const long long S = (long long)gridDim.x * NT;
  const int c = threadIdx.x % LPR;
  float wv[EPP], dwa[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) {
    wv[e] = p.w[c * EPP + e];
    dwa[e] = 0.f;
  }
  const i32x4* X = reinterpret_cast<const i32x4*>(p.x);
  const i32x4* Z = reinterpret_cast<const i32x4*>(p.z);
  const i32x4* DY = reinterpret_cast<const i32x4*>(p.dy);
  i32x4* DX = reinterpret_cast<i32x4*>(p.dx);
  i32x4* DZ = reinterpret_cast<i32x4*>(p.dz);
  const float inv_d = 1.f / (float)D;
  for (long long q0 = (long long)blockIdx.x * NT + threadIdx.x; q0 < npieces; q0 += PPT * S) {
    i32x4 xv[PPT], zv[PPT], gv[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {   // unconditional reads (piece 0 out of range): all in flight
      const long long q = q0 + k * S, qc = q < npieces ? q : 0;
      xv[k] = X[qc];
      zv[k] = Z[qc];
      gv[k] = DY[qc];
    }
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const long long q = q0 + k * S;
      const typename P::F xf = P::to_f(xv[k]), zf = P::to_f(zv[k]), gf = P::to_f(gv[k]);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) ss += xf[e] * xf[e];
      ss = row_sum<LPR>(ss);
      const float r = rsqrtf(ss * inv_d + p.eps);
      typename P::F n, dn, dzf;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        n[e] = xf[e] * r;
        const float s = sigmoid(zf[e]);
        const float a = n[e] * wv[e];
        const float da = gf[e] * (zf[e] * s);
        dzf[e] = gf[e] * a * s * (1.f + zf[e] * (1.f - s));
        if (q < npieces) dwa[e] += da * n[e];
        dn[e] = da * wv[e];
        dot += dn[e] * n[e];
      }
      dot = row_sum<LPR>(dot) * inv_d;
      typename P::F dxf;
#pragma unroll
      for (int e = 0; e < EPP; ++e) dxf[e] = r * (dn[e] - n[e] * dot);
      if (q < npieces) {
        DX[q] = P::from_f(dxf);
        DZ[q] = P::from_f(dzf);
      }
    }
  }
  // per-workgroup partial of dw: column c * EPP + e, summed over the threads
  // of this column block in thread order; stored column-major, part[col][wg]
#pragma unroll
  for (int e = 0; e < EPP; ++e) red[threadIdx.x * EPP + e] = dwa[e];
  __syncthreads();
  if (threadIdx.x < D) {
    const int col = threadIdx.x, cb = col / EPP, e = col - cb * EPP;
    float acc = 0.f;
    for (int j = 0; j < NT / LPR; ++j) acc += red[(j * LPR + cb) * EPP + e];
    p.part[(size_t)col * p.nblk + blockIdx.x] = acc;
  }
}

// dw[col] = the sum of column col's nblk partials, one wave per column: lane
// l adds partials l, l + 64, ... in order (all reads issued first), then a
// butterfly over the wave.
__global__ __launch_bounds__(64) void k_gnorm_dw(GnormParams p) {
  constexpr int PER = GNORM_MAX_BWD_BLOCKS / 64;
  const int col = blockIdx.x, l = threadIdx.x;
  const float* src = p.part + (size_t)col * p.nblk;
  float v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int b = l + 64 * k;
    v[k] = b < p.nblk ? src[b] : 0.f;
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) acc += v[k];
  acc = row_sum<64>(acc);
  if (l == 0) p.dw[col] = acc;
}

template <typename E, int D>
hipError_t gnorm_fwd_t(const GnormParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  GnormParams a = p;
  a.nblk = gnorm_blocks(p.rows, D, sizeof(E) == 2, false);
  void* args[] = {&a};
  return hipLaunchKernel((const void*)k_gnorm_fwd<E, D>, dim3(a.nblk), dim3(NT), args, 0, s);
}

template <typename E, int D>
hipError_t gnorm_bwd_t(const GnormParams& p, hipStream_t s) {
  GnormParams a = p;
  a.nblk = gnorm_blocks(p.rows, D, sizeof(E) == 2, true);
  if (a.nblk == 0) return hipSuccess;
  void* args[] = {&a};
  return hipLaunchKernel((const void*)k_gnorm_bwd<E, D>, dim3(a.nblk), dim3(NT), args, 0, s);
}

}  // namespace

int gnorm_blocks(long long rows, int D, bool bf16, bool bwd) {
  const long long lpr = (long long)D * (bf16 ? 2 : 4) / 16;
  const long long want = (rows * lpr + (long long)NT * PPT - 1) / ((long long)NT * PPT);
  const long long cap = bwd ? GNORM_MAX_BWD_BLOCKS : 65535;
  return (int)(want < cap ? want : cap);
}

hipError_t launch_gnorm_fwd(const GnormParams& p, int D, bool is_bf16, hipStream_t s) {
  if (D == 64) return is_bf16 ? gnorm_fwd_t<bf16, 64>(p, s) : gnorm_fwd_t<float, 64>(p, s);
  if (D == 128) return is_bf16 ? gnorm_fwd_t<bf16, 128>(p, s) : gnorm_fwd_t<float, 128>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gnorm_bwd(const GnormParams& p, int D, bool is_bf16, hipStream_t s) {
  if (D == 64) return is_bf16 ? gnorm_bwd_t<bf16, 64>(p, s) : gnorm_bwd_t<float, 64>(p, s);
  if (D == 128) return is_bf16 ? gnorm_bwd_t<bf16, 128>(p, s) : gnorm_bwd_t<float, 128>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gnorm_dw(const GnormParams& p, int D, bool is_bf16, hipStream_t s) {
  GnormParams a = p;
  a.nblk = gnorm_blocks(p.rows, D, is_bf16, true);
  void* args[] = {&a};
  return hipLaunchKernel((const void*)k_gnorm_dw, dim3(D), dim3(64), args, 0, s);
}

}  // namespace gdn
