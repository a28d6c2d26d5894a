// conv.hip -- causal depthwise conv1d (optional SiLU) over packed sequences,
// forward and backward.
//
// XTuner / Ascend 910C Qwen3.5 training article, §3.1.2: the GDN stack's
// causal conv1d, first a loop of slices and pads per sequence, then one
// native forward and one backward kernel (Fig. 8).  Per channel c, kernel
// size K <= 4, token t of a sequence whose first token is t0:
//     pre[t] = bias + sum_j w[j] x[t - (K-1) + j]   (x = 0 before t0)
//     y[t]   = silu(pre[t])  (or pre[t])
// and, for an upstream dy, dpre = dy silu'(pre) (or dy),
//     dx[t'] = sum_j w[j] dpre[t' + (K-1) - j]      (same sequence only)
//     dw[j]  = sum_t dpre[t] x[t - (K-1) + j],  dbias = sum_t dpre[t].
// All arithmetic fp32; each output rounded once.
//
// Layout: x, y, dy, dx are [tokens][C] (channels last); w is [C][K], bias
// [C], fp32.  A lane owns CPT = 4 consecutive channels (an 8-byte bf16 or
// 16-byte fp32 piece of a row), so a wave reads a contiguous run; a wave
// streams TW consecutive tokens through a register window of the last K inputs (and,
// backward, the last K values of dpre), so every row is read once plus a
// K-1 row halo.  Sequence boundaries enter only through each token's
// position in its sequence (pos) and the tokens left after it (rem): tap s
// of y[t] reads x[t - s] iff s <= pos(t), and dx[t'] takes dpre[t' + d] iff
// d <= rem(t').  A forward tile whose reach lies inside one sequence (nearly
// all of them) runs a copy of the body without these checks.  dw and dbias:
// per-lane sums over the lane's tokens, then a
// fixed-order sum over the waves of a workgroup (one partial per workgroup
// row of the grid) and, in k_conv_dw, over the partials.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "frag.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int NW = 4;     // waves per workgroup (token sub-tiles)
// Tokens per wave: longer tiles cut the halo re-reads (the backward's is
// two-sided), shorter ones give a narrow problem (few channels) enough waves.
// The launcher picks per problem.
constexpr int TWF = 16, TWF_NARROW = 8;    // forward
constexpr int TWB = 32, TWB_NARROW = 16;   // backward
constexpr long long FWD_MIN_WG = 1536, BWD_MIN_WG = 768;   // 6 and 3 workgroups per CU

__host__ __device__ constexpr long long cdiv(long long a, long long b) { return (a + b - 1) / b; }
inline int conv_gx(int C) { return (C / 4 + 63) / 64; }
inline int conv_fwd_tw(long long tokens, int C) {
  return conv_gx(C) * cdiv(tokens, NW * TWF) >= FWD_MIN_WG ? TWF : TWF_NARROW;
}
inline int conv_bwd_tw(long long tokens, int C) {
  const long long rows = cdiv(tokens, NW * TWB);
  return conv_gx(C) * (rows < CONV_MAX_BWD_ROWS ? rows : CONV_MAX_BWD_ROWS) >= BWD_MIN_WG ? TWB : TWB_NARROW;
}

// A lane's piece of a row: N channels, raw as stored (R) and in fp32 (F).
template <typename E, int N> struct CPiece;
template <> struct CPiece<bf16, 4> {
  using R = bf16x4;
  using F = f32x4;
  static __device__ __forceinline__ F to_f(R v) { return __builtin_convertvector(v, f32x4); }
  static __device__ __forceinline__ R from_f(F f) { return __builtin_convertvector(f, bf16x4); }
};
template <> struct CPiece<float, 4> {
  using R = f32x4;
  using F = f32x4;
  static __device__ __forceinline__ F to_f(R v) { return v; }
  static __device__ __forceinline__ R from_f(F f) { return f; }
};

__device__ __forceinline__ float csigmoid(float u) { return __builtin_amdgcn_rcpf(1.f + __expf(-u)); }

// Position of token t in its sequence and the tokens after it (rem); tokens
// past the end get pos = rem = -1 (never read, never contribute).
__device__ __forceinline__ void seq_pos(const ConvParams& p, long long t, int& pos, int& rem) {
  if (t < 0 || t >= p.tokens) {
    pos = rem = -1;
    return;
  }
  if (!p.cu) {
    const long long q = t / p.dense_T;
    pos = (int)(t - q * p.dense_T);
    rem = p.dense_T - 1 - pos;
    return;
  }
  // the last sequence n with cu[n] <= t (empty sequences are skipped by it)
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  pos = (int)(t - p.cu[lo]);
  rem = (int)(p.cu[lo + 1] - 1 - t);
}

// Row t's piece cp, or zeros outside the tokens / channels.  The read is
// unconditional (from row 0, piece 0 when out of range; tokens >= 1), so a
// batch of these issues back to back instead of one branch and wait each.
// CHECK = false: the caller knows 0 <= t < tokens.
template <typename E, int CPT, bool CHECK = true>
__device__ __forceinline__ typename CPiece<E, CPT>::R load_row(const ConvParams& p, const void* base, long long t, int cp, bool live) {
  using R = typename CPiece<E, CPT>::R;
  const bool ok = CHECK ? live && t >= 0 && t < p.tokens : live;
  const R v = reinterpret_cast<const R*>(base)[(ok ? t : 0) * (p.C / CPT) + (ok ? cp : 0)];
  return ok ? v : R{};
}

template <typename E, int K, int CPT, int TW>
__global__ __launch_bounds__(64 * NW) void k_conv_fwd(ConvParams p) {
  using P = CPiece<E, CPT>;
  using F = typename P::F;
  constexpr int WIN = TW + 6;   // (pos, rem) of tokens t_a - 3 .. t_a + TW + 2
  const int lane = lane_id(), w = wave_id();
  const int cp = blockIdx.x * 64 + lane;        // channel piece of this lane
  const bool live = cp * CPT < p.C;
  float wt[K][CPT], bs[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    const int c = live ? cp * CPT + e : 0;
#pragma unroll
    for (int j = 0; j < K; ++j) wt[j][e] = p.w[(size_t)c * K + j];
    bs[e] = p.bias ? p.bias[c] : 0.f;
  }
  typename P::R* Y = reinterpret_cast<typename P::R*>(p.y);
  // one tile of TW tokens starting at ta; INNER: no sequence boundary in reach
  auto fwd_tile = [&](auto inner_c, long long ta, int pv) {
    constexpr bool INNER = decltype(inner_c)::value;
    F hist[4];   // x[t], x[t-1], x[t-2], x[t-3] once the step's shift is done
    hist[3] = F{};
#pragma unroll
    for (int s = 1; s < 4; ++s) hist[s - 1] = P::to_f(load_row<E, CPT>(p, p.x, ta - s, cp, live && s < K));
#pragma unroll
    for (int i0 = 0; i0 < TW; i0 += 8) {
      typename P::R xs[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xs[i] = load_row<E, CPT, !INNER>(p, p.x, ta + i0 + i, cp, live);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const long long t = ta + i0 + i;
        hist[3] = hist[2];
        hist[2] = hist[1];
        hist[1] = hist[0];
        hist[0] = P::to_f(xs[i]);
        const int pos = __builtin_amdgcn_readlane(pv, i0 + i + 3);
        if (!INNER && t >= p.tokens) continue;
        F o;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          float acc = bs[e];
#pragma unroll
          for (int s = 0; s < K; ++s)
            if (INNER || s <= pos) acc += wt[K - 1 - s][e] * hist[s][e];
          o[e] = p.act ? acc * csigmoid(acc) : acc;
        }
        if (live) Y[t * (p.C / CPT) + cp] = P::from_f(o);
      }
    }
  };
  for (long long tile = blockIdx.y; tile * (NW * TW) < p.tokens; tile += gridDim.y) {
    const long long ta = tile * (NW * TW) + (long long)w * TW;
    if (ta >= p.tokens) break;
    // (pos, rem) of tokens ta - 3 + l in lane l
    int pv = -1, rv = -1;
    if (lane < WIN) seq_pos(p, ta - 3 + lane, pv, rv);
    // tokens ta - 3 .. ta + TW - 1 in one sequence (so inside the tokens): no
    // tap of the tile crosses a boundary, and the body runs without checks
    if (__builtin_amdgcn_readlane(pv, TW + 2) >= TW + 2) fwd_tile(std::true_type{}, ta, pv);
    else fwd_tile(std::false_type{}, ta, pv);
  }
}

template <typename E, int K, int TW>
__global__ __launch_bounds__(64 * NW) void k_conv_bwd(ConvParams p) {
  constexpr int CPT = 4;
  using P = CPiece<E, CPT>;
  constexpr int WIN = TW + 6;   // (pos, rem) of tokens t_a - 3 .. t_a + TW + 2
  constexpr int NP = CPT * (K + 1);   // per-lane partial sums: dw taps, then dbias
  __shared__ float red[NW][64][NP];
  const int lane = lane_id(), w = wave_id();
  const int cp = blockIdx.x * 64 + lane;
  const bool live = cp * CPT < p.C;
  float wt[K][CPT], bs[CPT], acc_w[K][CPT], acc_b[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    const int c = live ? cp * CPT + e : 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      wt[j][e] = p.w[(size_t)c * K + j];
      acc_w[j][e] = 0.f;
    }
    bs[e] = p.bias ? p.bias[c] : 0.f;
    acc_b[e] = 0.f;
  }
  typename P::R* DX = reinterpret_cast<typename P::R*>(p.dx);
  for (long long tile = blockIdx.y; tile * (NW * TW) < p.tokens; tile += gridDim.y) {
    const long long ta = tile * (NW * TW) + (long long)w * TW;
    if (ta >= p.tokens) continue;   // no barrier inside the loop: waves may leave early
    int pv = -1, rv = -1;
    if (lane < WIN) seq_pos(p, ta - 3 + lane, pv, rv);
    f32x4 xh[4];    // x[t], x[t-1], x[t-2], x[t-3] once the step's shift is done
    f32x4 dh[4];    // dpre[t], dpre[t-1], dpre[t-2], dpre[t-3] likewise (dpre before ta is never used)
    xh[3] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) dh[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 1; s < 4; ++s) xh[s - 1] = P::to_f(load_row<E, CPT>(p, p.x, ta - s, cp, live && s < K));
    // steps t = ta .. ta + TW + K - 2: dpre[t]; dx[t - (K-1)] once its window is complete
#pragma unroll
    for (int i0 = 0; i0 < TW + 8; i0 += 8) {
      typename P::R xs[8], gs[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool need = i0 + i < TW + K - 1;
        xs[i] = load_row<E, CPT>(p, p.x, ta + i0 + i, cp, live && need);
        gs[i] = load_row<E, CPT>(p, p.dy, ta + i0 + i, cp, live && need);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ii = i0 + i;
        if (ii >= TW + K - 1) continue;
        const long long t = ta + ii;
        xh[3] = xh[2];
        xh[2] = xh[1];
        xh[1] = xh[0];
        xh[0] = P::to_f(xs[i]);
        dh[3] = dh[2];
        dh[2] = dh[1];
        dh[1] = dh[0];
        const int pos = __builtin_amdgcn_readlane(pv, ii + 3);
        // dpre[t] (zero past the end of the tokens: pos = -1 there, and dy reads as zero)
        const f32x4 gf = P::to_f(gs[i]);
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          float pre = bs[e];
#pragma unroll
          for (int s = 0; s < K; ++s)
            if (s <= pos) pre += wt[K - 1 - s][e] * xh[s][e];
          float g = gf[e];
          if (p.act) {
            const float sg = csigmoid(pre);
            g = g * sg * (1.f + pre * (1.f - sg));
          }
          dh[0][e] = pos >= 0 ? g : 0.f;
        }
        // this wave's own tokens feed dw and dbias
        if (ii < TW && pos >= 0) {
#pragma unroll
          for (int e = 0; e < CPT; ++e) {
            acc_b[e] += dh[0][e];
#pragma unroll
            for (int s = 0; s < K; ++s)
              if (s <= pos) acc_w[K - 1 - s][e] += dh[0][e] * xh[s][e];
          }
        }
        // dx[t'] with t' = t - (K-1), over dpre[t' .. t]
        const int jj = ii - (K - 1);
        if (jj >= 0 && jj < TW) {
          const long long tp = t - (K - 1);
          const int rem = __builtin_amdgcn_readlane(rv, jj + 3);
          if (tp < p.tokens) {
            f32x4 o;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
              float a = 0.f;
#pragma unroll
              for (int d = 0; d < K; ++d)   // dpre[t' + d] sits in dh[K-1-d]
                if (d <= rem) a += wt[K - 1 - d][e] * dh[K - 1 - d][e];
              o[e] = a;
            }
            if (live) DX[tp * (p.C / CPT) + cp] = P::from_f(o);
          }
        }
      }
    }
  }
  // partials of this workgroup: the waves' sums added in wave order
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
#pragma unroll
    for (int j = 0; j < K; ++j) red[w][lane][j * CPT + e] = acc_w[j][e];
    red[w][lane][K * CPT + e] = acc_b[e];
  }
  __syncthreads();
  if (w == 0 && live) {
    float* dst = p.part + (size_t)blockIdx.y * p.C * (K + 1);
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int c = cp * CPT + e;
#pragma unroll
      for (int j = 0; j <= K; ++j) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += red[ww][lane][j * CPT + e];
        dst[(size_t)c * (K + 1) + j] = s;   // [row of the grid][channel][tap | bias]
      }
    }
  }
}

// dw[c][j] (j < K) and dbias[c] (j = K): the sum over the grid rows' partials in
// row order, one thread per (channel, tap).
__global__ __launch_bounds__(256) void k_conv_dw(ConvParams p) {
  const int K1 = p.K + 1;
  const long long n = (long long)p.C * K1;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float s = 0.f;
  for (int r0 = 0; r0 < p.ntiles; r0 += 16) {   // 16 reads in flight, added in row order
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = r0 + i < p.ntiles ? p.part[(size_t)(r0 + i) * n + e] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += v[i];
  }
  const int c = (int)(e / K1), j = (int)(e - (long long)c * K1);
  if (j < p.K) p.dw[(size_t)c * p.K + j] = s;
  else if (p.dbias) p.dbias[c] = s;
}

template <typename E, int K>
hipError_t conv_fwd_t(const ConvParams& p, hipStream_t s) {
  if (p.tokens == 0 || p.C == 0) return hipSuccess;
  ConvParams a = p;
  void* args[] = {&a};
  // 4 channels per lane: 16-byte bf16 pieces (8 channels) measured slower,
  // the grid has half the waves
  const int tw = conv_fwd_tw(p.tokens, p.C);
  const long long tiles = cdiv(p.tokens, NW * tw);
  const int gy = (int)(tiles < 65535 ? tiles : 65535);
  const void* k = tw == TWF ? (const void*)k_conv_fwd<E, K, 4, TWF> : (const void*)k_conv_fwd<E, K, 4, TWF_NARROW>;
  return hipLaunchKernel(k, dim3(conv_gx(p.C), gy), dim3(64 * NW), args, 0, s);
}

template <typename E, int K>
hipError_t conv_bwd_t(const ConvParams& p, hipStream_t s) {
  ConvParams a = p;
  a.ntiles = conv_bwd_rows(p.tokens, p.C);
  void* args[] = {&a};
  if (p.tokens > 0 && p.C > 0) {
    const void* k = conv_bwd_tw(p.tokens, p.C) == TWB ? (const void*)k_conv_bwd<E, K, TWB>
                                                       : (const void*)k_conv_bwd<E, K, TWB_NARROW>;
    hipError_t e = hipLaunchKernel(k, dim3(conv_gx(p.C), a.ntiles), dim3(64 * NW), args, 0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename E>
hipError_t conv_fwd_e(const ConvParams& p, hipStream_t s) {
  switch (p.K) {
    case 1: return conv_fwd_t<E, 1>(p, s);
    case 2: return conv_fwd_t<E, 2>(p, s);
    case 3: return conv_fwd_t<E, 3>(p, s);
    case 4: return conv_fwd_t<E, 4>(p, s);
  }
  return hipErrorInvalidValue;
}
template <typename E>
hipError_t conv_bwd_e(const ConvParams& p, hipStream_t s) {
  switch (p.K) {
    case 1: return conv_bwd_t<E, 1>(p, s);
    case 2: return conv_bwd_t<E, 2>(p, s);
    case 3: return conv_bwd_t<E, 3>(p, s);
    case 4: return conv_bwd_t<E, 4>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int conv_bwd_rows(long long tokens, int C) {
  const long long tiles = cdiv(tokens, NW * conv_bwd_tw(tokens, C));
  if (tiles <= 0) return 0;
  return (int)(tiles < CONV_MAX_BWD_ROWS ? tiles : CONV_MAX_BWD_ROWS);
}

hipError_t launch_conv_fwd(const ConvParams& p, bool is_bf16, hipStream_t s) {
  return is_bf16 ? conv_fwd_e<bf16>(p, s) : conv_fwd_e<float>(p, s);
}

hipError_t launch_conv_bwd(const ConvParams& p, bool is_bf16, hipStream_t s) {
  return is_bf16 ? conv_bwd_e<bf16>(p, s) : conv_bwd_e<float>(p, s);
}

hipError_t launch_conv_dw(const ConvParams& p, hipStream_t s) {
  ConvParams a = p;
  a.ntiles = conv_bwd_rows(p.tokens, p.C);
  void* args[] = {&a};
  const long long n = (long long)p.C * (p.K + 1);
  if (n == 0) return hipSuccess;
  return hipLaunchKernel((const void*)k_conv_dw, dim3((unsigned)((n + 255) / 256)), dim3(256), args, 0, s);
}

}  // namespace gdn
