// tri.h -- T = (I + A)^-1 for a 64x64 strictly lower A in fp32, in LDS,
// with 16x16x4 fp32 MFMAs (the intra-chunk triangular solve).
//
// 16x16 blocks (a, b), a >= b.  Diagonal blocks use the exact product form
// for a nilpotent matrix (A_bb^16 = 0):
//     T_bb = (I - A)(I + A^2)(I + A^4)(I + A^8),          A = A_bb,
// computed in registers: a 16x16 accumulator of X read by lane l as
// X[4 lg + q][li] is the B operand of a product as it stands and the A
// operand of the transposed product, so each intermediate is carried in
// both orientations and the chain needs no LDS traffic.  Off-diagonal
// blocks follow by levels (forward substitution on blocks):
//     T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb.
#pragma once
#include "frag.h"

namespace gdn {

// acc += sum_k X[k][m] Y[k][n] where lane l holds X[4lg+e][li] in x[e]
// and Y[4lg+e][li] in y[e] (both accumulator layout): the product X^T Y.
__device__ __forceinline__ f32x4 mm16_tt(f32x4 x, f32x4 y, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e], y[e], acc, 0, 0, 0);
  return acc;
}

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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, li = lane & 15, lg = lane >> 4;
  zero_off_blocks<float, true>(T, ld, threadIdx.x, 64 * nw);
  // diagonal blocks
  for (int b = w; b < 4; b += nw) {
    const int o = 16 * b;
    // A (accumulator layout) and A^T, masked to the strict lower triangle, rows scaled
    f32x4 A, At;
    {
      const f32x4 a = acc16(M, ld, o, o, li, lg);   // M[o+4lg+q][o+li]
      const f32x4 t = rows16(M, ld, o, o, li, lg);  // M[o+li][o+4lg+q]
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * lg + q;  // row of a / column index of t
        const float sr = rs ? rs[o + r] : 1.f, sl = rs ? rs[o + li] : 1.f;
        A[q] = li < r ? sr * a[q] : 0.f;           // A[r][li]
        At[q] = r < li ? sl * t[q] : 0.f;          // A^T[r][li] = A[li][r]
      }
    }
    f32x4 I;
#pragma unroll
    for (int q = 0; q < 4; ++q) I[q] = (4 * lg + q == li) ? 1.f : 0.f;
    const f32x4 z = zero4();
    // powers: P1 = A^2, P2 = A^4, P3 = A^8 (and transposes)
    const f32x4 P1 = mm16_tt(At, A, z), P1t = mm16_tt(A, At, z);
    const f32x4 P2 = mm16_tt(P1t, P1, z), P2t = mm16_tt(P1, P1t, z);
    const f32x4 P3 = mm16_tt(P2t, P2, z);
    // F1 = (I - A)(I + P1) = I - A + P1 - A P1
    const f32x4 AP1 = mm16_tt(At, P1, z), AP1t = mm16_tt(P1, At, z);
    const f32x4 F1 = I - A + P1 - AP1, F1t = I - At + P1t - AP1t;
    // F2 = F1 (I + P2)
    const f32x4 F2 = F1 + mm16_tt(F1t, P2, z), F2t = F1t + mm16_tt(P2, F1t, z);
    // T = F2 (I + P3)
    const f32x4 Tb = F2 + mm16_tt(F2t, P3, z);
    store_acc16(T, ld, o, o, li, lg, Tb);
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
