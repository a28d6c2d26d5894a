// tri.h -- T = (I + A)^-1 for a 64x64 strictly lower A in fp32, in LDS
// (the intra-chunk triangular solve).
//
// 16x16 blocks (a, b), a >= b.  Each diagonal block is inverted by forward
// substitution over its four 4-row groups, entirely in the VALU: lane l
// (li = l % 16, lg = l / 16) owns column li of the block and rows 4 lg .. 4 lg
// + 3, i.e. it ends holding T_bb in the 16x16 accumulator layout.  Row group
// H is finished at step H: its residual rows are fetched from lane group H by
// a lane shuffle, the 4x4 unit-lower system (I + A_HH) y = residual is solved
// in every lane, and the later row groups subtract A_GH y.  Every value is a
// plain substitution result, so the rounding error stays that of forward
// substitution when entries of A approach 1 (an explicit product of powers of
// A, e.g. (I - A)(I + A^2)(I + A^4)(I + A^8), would form entries far larger
// than T's and lose digits to cancellation).  Off-diagonal blocks follow by
// levels (forward substitution on blocks) with 16x16x4 fp32 MFMAs:
//     T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb.
#pragma once
#include "frag.h"

namespace gdn {

// Row block of a row-major LDS matrix as an A operand: lane gets M[r0+li][c0+4lg+e].
__device__ __forceinline__ f32x4 rows16(const float* M, int ld, int r0, int c0, int li, int lg) {
  return *reinterpret_cast<const f32x4*>(M + (r0 + li) * ld + c0 + 4 * lg);
}
// Block in accumulator layout: lane gets M[r0+4lg+e][c0+li].
__device__ __forceinline__ f32x4 acc16(const float* M, int ld, int r0, int c0, int li, int lg) {
  const float* p = M + (r0 + 4 * lg) * ld + c0 + li;
  return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}
__device__ __forceinline__ void store_acc16(float* M, int ld, int r0, int c0, int li, int lg, f32x4 v) {
  float* p = M + (r0 + 4 * lg) * ld + c0 + li;
  p[0] = v[0];
  p[ld] = v[1];
  p[2 * ld] = v[2];
  p[3 * ld] = v[3];
}

// T = (I + A)^-1 where A[r][s] = rs[r] * M[r][s] for s < r (rs = nullptr
// means 1).  M: strictly lower part read only.  T: full 64x64 written (upper
// zero).  All `nw` waves of the workgroup call this; it ends with a barrier.
__device__ inline void tri_inverse64(const float* M, const float* rs, float* T, int ld, int nw) {
  const int lane = lane_id(), w = wave_id(), li = lane & 15, lg = lane >> 4;
  zero_off_blocks<float, true>(T, ld, threadIdx.x, 64 * nw);
  // diagonal blocks: lane (li, lg) solves column li, row group lg
  for (int b = w; b < 4; b += nw) {
    const int o = 16 * b;
    f32x4 r, x = zero4();   // residual and result rows o + 4 lg + q of column o + li
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = (4 * lg + q == li) ? 1.f : 0.f;
#pragma unroll
    for (int H = 0; H < 4; ++H) {
      // the residual of row group H in this column (held by lane group H)
      f32x4 y;
#pragma unroll
      for (int q = 0; q < 4; ++q) y[q] = __shfl(r[q], li + 16 * H, 64);
      // (I + A_HH) y = residual; A_HH is the same in every lane
#pragma unroll
      for (int q = 1; q < 4; ++q) {
        const float* arow = M + (o + 4 * H + q) * ld + o + 4 * H;
        const float sr = rs ? rs[o + 4 * H + q] : 1.f;
#pragma unroll
        for (int qq = 0; qq < q; ++qq) y[q] -= (sr * arow[qq]) * y[qq];
      }
      if (lg == H) x = y;
      if (H < 3) {
        // later row groups take this group's part: r -= A_{lg,H} y
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(M + (o + 4 * lg + q) * ld + o + 4 * H);
          const float sr = rs ? rs[o + 4 * lg + q] : 1.f;
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) t += (sr * a[e]) * y[e];
          if (lg > H) r[q] -= t;
        }
      }
    }
    store_acc16(T, ld, o, o, li, lg, x);
  }
  __syncthreads();
  // off-diagonal blocks by level d = a - b
  for (int d = 1; d < 4; ++d) {
    for (int a = d + w; a < 4; a += nw) {
      const int b = a - d;
      f32x4 X = zero4();
      for (int c = b; c < a; ++c) {
        // X += A_ac T_cb : A operand rows of A_ac (scaled), B operand T_cb (accumulator layout)
        f32x4 ar = rows16(M, ld, 16 * a, 16 * c, li, lg);
        const float sr = rs ? rs[16 * a + li] : 1.f;
        ar = scale4(ar, sr);
        const f32x4 tc = acc16(T, ld, 16 * c, 16 * b, li, lg);
#pragma unroll
        for (int e = 0; e < 4; ++e) X = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[e], tc[e], X, 0, 0, 0);
      }
      // T_ab = -T_aa X
      const f32x4 ta = rows16(T, ld, 16 * a, 16 * a, li, lg);
      f32x4 Y = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) Y = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[e], X[e], Y, 0, 0, 0);
      store_acc16(T, ld, 16 * a, 16 * b, li, lg, -Y);
    }
    __syncthreads();
  }
}

}  // namespace gdn
