// recur.hip -- the gated delta rule token by token, for decoding: a few new
// tokens per sequence, the state read and written once per call (in place).
//
// XTuner / Ascend 910C Qwen3.5 training article, §3.1.2: the operator whose
// chunked kernels the rest of this library implements.  The pages cover
// training only; this is the same recurrence, written for the shape regime
// where each sequence brings a handful of tokens.  With the state as h = S^T
// ([d_k][d_v], h[i][j] = S[j][i]) each token t is
//     a = exp(g_t),  r = h^T k_t,  u = beta_t (v_t - a r),
//     h <- a h + k_t u^T,           o_t = scale h^T q_t
// (S_t = a S_{t-1} (I - beta k k^T) + beta v k^T, o_t = scale S_t q_t).
//
// One workgroup per (sequence, head) holds h in registers for the whole call,
// each thread a 16 x 4 block of it; q_t and k_t (normalised if asked) are
// staged in LDS and read by every thread.  HBM traffic: the state once each
// way plus the tokens' q, k, v, o.
#include <hip/hip_runtime.h>

#include "frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename E> __device__ __forceinline__ float ld(const void* p, size_t i) {
  return (float)reinterpret_cast<const E*>(p)[i];
}

// Thread (rg, cg) holds rows 16 rg .. 16 rg + 15 and columns 4 cg .. 4 cg + 3 of
// h: its state moves in 16-byte pieces, sixteen reads in flight at once.  The
// column sums h^T k and h^T q are per-thread partials over its rows, added
// across the row groups of a wave by a lane butterfly (bitwise the same in
// every lane) and across the waves through LDS in wave order.
template <typename E, int DK, int DV, bool NORM>
__global__ __launch_bounds__(DK * DV / 64) void k_recurrent(RecParams p) {
  constexpr int CG = DV / 4;        // column groups of 4
  constexpr int RG = DK / 16;       // row groups of 16
  constexpr int NT = CG * RG;       // threads
  constexpr int NWV = NT / 64;      // waves
  static_assert(NT % 64 == 0 && 64 % CG == 0 && NT >= DK, "thread layout");
  __shared__ float sq[DK], sk[DK];
  __shared__ f32x4 s_part[2][NWV][CG];
  __shared__ float s_red[2][NWV];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cg = tid % CG, rg = tid / CG;
  const int n = blockIdx.x / p.H, hh = blockIdx.x - n * p.H;
  long long t0, t1;
  if (p.cu) {
    // clamped to the tokens the host copy describes, so a device copy that
    // differs from it cannot send the reads and writes outside the tensors
    t0 = min(max((long long)p.cu[n], 0LL), p.tokens);
    t1 = min(max((long long)p.cu[n + 1], t0), p.tokens);
  } else {
    t0 = (long long)n * p.dense_T;
    t1 = t0 + p.dense_T;
  }
  quad_t<E>* O = reinterpret_cast<quad_t<E>*>(p.o);
  const long long slot = p.idx ? (long long)p.idx[n] : (long long)n;
  if (slot < 0 || slot >= p.num_slots) {
    // no state for this sequence: its outputs are zero, no state is touched
    if (rg == 0)
      for (long long t = t0; t < t1; ++t) O[(((size_t)t * p.H + hh) * DV) / 4 + cg] = to_quad<E>(zero4());
    return;
  }
  // the (slot, head) block of the state: a uniform base and 32-bit offsets
  float* st = p.state + ((size_t)__builtin_amdgcn_readfirstlane((int)slot) * p.H + hh) * DK * DV;
  f32x4 h[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) h[r] = *reinterpret_cast<const f32x4*>(st + (16 * rg + r) * DV + 4 * cg);
  // the sum over all row groups of a per-thread column partial
  auto col_sum = [&](f32x4 x, int which) {
#pragma unroll
    for (int off = CG; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += __shfl_xor(x[e], off, 64);
    if constexpr (NWV > 1) {
      if (lane < CG) s_part[which][wv][cg] = x;
      __syncthreads();
      x = s_part[which][0][cg];
#pragma unroll
      for (int w = 1; w < NWV; ++w) x = x + s_part[which][w][cg];
    }
    return x;
  };
  for (long long t = t0; t < t1; ++t) {
    const size_t th = (size_t)t * p.H + hh;
    if (tid < DK) {
      sq[tid] = ld<E>(p.q, (size_t)t * p.ldq + (size_t)hh * DK + tid);
      sk[tid] = ld<E>(p.k, (size_t)t * p.ldq + (size_t)hh * DK + tid);
    }
    const float a = __expf(p.g[th]);
    const float b = p.beta[th];
    const f32x4 vj = quad_to_f32<E>(*reinterpret_cast<const quad_t<E>*>(reinterpret_cast<const E*>(p.v) + (size_t)t * p.ldv + (size_t)hh * DV + 4 * cg));
    __syncthreads();
    float iq = 1.f, ik = 1.f;
    if constexpr (NORM) {
      // reciprocal norms y = x / max(||x||, 1e-12): per-wave sums, then the waves in order
      float a2 = tid < DK ? sq[tid] * sq[tid] : 0.f, b2 = tid < DK ? sk[tid] * sk[tid] : 0.f;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        a2 += __shfl_xor(a2, off, 64);
        b2 += __shfl_xor(b2, off, 64);
      }
      if (lane == 0) {
        s_red[0][wv] = a2;
        s_red[1][wv] = b2;
      }
      __syncthreads();
      float nq = 0.f, nk = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        nq += s_red[0][w];
        nk += s_red[1][w];
      }
      iq = 1.f / fmaxf(sqrtf(nq), 1e-12f);
      ik = 1.f / fmaxf(sqrtf(nk), 1e-12f);
    }
    // r = h^T k over this thread's rows, then over all rows
    f32x4 rp = zero4();
#pragma unroll
    for (int r = 0; r < 16; ++r) rp = rp + h[r] * sk[16 * rg + r];
    const f32x4 rr = col_sum(rp, 0);
    f32x4 u;   // beta (v - a r) with k entering the update as ik * k
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = b * (vj[e] - a * rr[e] * ik) * ik;
    // the rank-one update of this thread's block and its part of h^T q
    f32x4 op = zero4();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      h[r] = a * h[r] + sk[16 * rg + r] * u;
      op = op + h[r] * sq[16 * rg + r];
    }
    const f32x4 oo = col_sum(op, 1);
    if (rg == 0) O[(th * DV) / 4 + cg] = to_quad<E>(oo * (p.scale * iq));
    __syncthreads();   // sq, sk, s_part are rewritten by the next token
  }
  // written back non-temporal: the next reader is the next call, and a state
  // pool of this size would otherwise be evicted from the caches (written
  // back) in the middle of that call's reads
#pragma unroll
  for (int r = 0; r < 16; ++r)
    __builtin_nontemporal_store(h[r], reinterpret_cast<f32x4*>(st + (16 * rg + r) * DV + 4 * cg));
}

template <typename E, int DK, int DV>
hipError_t rec_t(const RecParams& p, hipStream_t s) {
  if (p.N * p.H == 0) return hipSuccess;
  RecParams a = p;
  void* args[] = {&a};
  const void* k = p.norm ? (const void*)k_recurrent<E, DK, DV, true> : (const void*)k_recurrent<E, DK, DV, false>;
  return hipLaunchKernel(k, dim3((unsigned)(p.N * p.H)), dim3(DK * DV / 64), args, 0, s);
}

template <typename E>
hipError_t rec_e(const RecParams& p, int dk, int dv, hipStream_t s) {
  if (dk == 64 && dv == 64) return rec_t<E, 64, 64>(p, s);
  if (dk == 64 && dv == 128) return rec_t<E, 64, 128>(p, s);
  if (dk == 128 && dv == 64) return rec_t<E, 128, 64>(p, s);
  if (dk == 128 && dv == 128) return rec_t<E, 128, 128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_recurrent(const RecParams& p, int dk, int dv, bool is_bf16, hipStream_t s) {
  return is_bf16 ? rec_e<bf16>(p, dk, dv, s) : rec_e<float>(p, dk, dv, s);
}

}  // namespace gdn
