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
// The columns of h are independent, so one workgroup per (sequence, head)
// gives thread j the column j of h, its d_k values in registers for the whole
// call; q_t and k_t (normalised if asked) are staged in LDS and read by every
// thread.  HBM traffic: the state once each way plus the tokens' q, k, v, o.
#include <hip/hip_runtime.h>

#include "frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename E> __device__ __forceinline__ float ld(const void* p, size_t i) {
  return (float)reinterpret_cast<const E*>(p)[i];
}

template <typename E, int DK, int DV, bool NORM>
__global__ __launch_bounds__(DV) void k_recurrent(RecParams p) {
  constexpr int NWV = DV / 64;
  __shared__ float sq[DK], sk[DK];
  __shared__ float s_red[2][NWV];
  const int n = blockIdx.x / p.H, hh = blockIdx.x - n * p.H;
  const int j = threadIdx.x;
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
  const long long slot = p.idx ? (long long)p.idx[n] : (long long)n;
  if (slot < 0 || slot >= p.num_slots) {
    // no state for this sequence: its outputs are zero, no state is touched
    for (long long t = t0; t < t1; ++t) {
      E* o = reinterpret_cast<E*>(p.o);
      o[((size_t)t * p.H + hh) * DV + j] = (E)0.f;
    }
    return;
  }
  // the (slot, head) block of the state: a uniform base and 32-bit offsets, so
  // the d_k reads and writes of a thread need no address registers each
  float* st = p.state + ((size_t)__builtin_amdgcn_readfirstlane((int)slot) * p.H + hh) * DK * DV;
  float h[DK];
#pragma unroll
  for (int i = 0; i < DK; ++i) h[i] = st[i * DV + j];
  for (long long t = t0; t < t1; ++t) {
    const size_t th = (size_t)t * p.H + hh;
    for (int i = j; i < DK; i += DV) {
      sq[i] = ld<E>(p.q, (size_t)t * p.ldq + (size_t)hh * DK + i);
      sk[i] = ld<E>(p.k, (size_t)t * p.ldq + (size_t)hh * DK + i);
    }
    const float a = __expf(p.g[th]);
    const float b = p.beta[th];
    const float vj = ld<E>(p.v, (size_t)t * p.ldv + (size_t)hh * DV + j);
    __syncthreads();
    float iq = 1.f, ik = 1.f;
    if constexpr (NORM) {
      // reciprocal norms y = x / max(||x||, 1e-12): per-wave partial sums, then the waves in order
      float a2 = 0.f, b2 = 0.f;
      for (int i = j; i < DK; i += DV) {
        a2 += sq[i] * sq[i];
        b2 += sk[i] * sk[i];
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        a2 += __shfl_xor(a2, off, 64);
        b2 += __shfl_xor(b2, off, 64);
      }
      if ((j & 63) == 0) {
        s_red[0][j >> 6] = a2;
        s_red[1][j >> 6] = b2;
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
    // r = h^T k (four partial chains), then the rank-one update and the output
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
#pragma unroll
    for (int i = 0; i < DK; i += 4) {
      r0 += h[i] * sk[i];
      r1 += h[i + 1] * sk[i + 1];
      r2 += h[i + 2] * sk[i + 2];
      r3 += h[i + 3] * sk[i + 3];
    }
    const float r = ((r0 + r1) + (r2 + r3)) * ik;
    const float u = b * (vj - a * r) * ik;   // k enters the update as ik * k
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
#pragma unroll
    for (int i = 0; i < DK; i += 4) {
      h[i] = a * h[i] + sk[i] * u;
      h[i + 1] = a * h[i + 1] + sk[i + 1] * u;
      h[i + 2] = a * h[i + 2] + sk[i + 2] * u;
      h[i + 3] = a * h[i + 3] + sk[i + 3] * u;
      o0 += h[i] * sq[i];
      o1 += h[i + 1] * sq[i + 1];
      o2 += h[i + 2] * sq[i + 2];
      o3 += h[i + 3] * sq[i + 3];
    }
    E* o = reinterpret_cast<E*>(p.o);
    o[th * DV + j] = (E)(p.scale * iq * ((o0 + o1) + (o2 + o3)));
    __syncthreads();   // sq, sk are rewritten by the next token
  }
  // written back non-temporal: the next reader is the next call, and a state
  // pool of this size would otherwise be evicted from the caches (written
  // back) in the middle of that call's reads
#pragma unroll
  for (int i = 0; i < DK; ++i) __builtin_nontemporal_store(h[i], st + i * DV + j);
}

template <typename E, int DK, int DV>
hipError_t rec_t(const RecParams& p, hipStream_t s) {
  if (p.N * p.H == 0) return hipSuccess;
  RecParams a = p;
  void* args[] = {&a};
  const void* k = p.norm ? (const void*)k_recurrent<E, DK, DV, true> : (const void*)k_recurrent<E, DK, DV, false>;
  return hipLaunchKernel(k, dim3((unsigned)(p.N * p.H)), dim3(DV), args, 0, s);
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
