// peak.hip -- measured peaks of one MI355X (gfx950), the ceilings beside the
// vendor figures that the operator's kernels are reported against:
//   - dense bf16 matrix-core rate: every wave issues a long run of
//     v_mfma_f32_16x16x32_bf16 on eight independent accumulators (no memory
//     traffic inside the loop);
//   - HBM bandwidth: a streaming copy and a streaming read of large buffers,
//     16 bytes per lane per access, grid-stride, enough waves to fill the chip.
//   - one wave's LDS read issue: the shader-clock cycles one wave spends per
//     1 KiB ds_read_b128 (64 lanes x 16 bytes, contiguous, no bank conflicts)
//     with many in flight, alone and with one MFMA issued after each read
//     (the pattern of the state passes' chunk step).
// Diagnostics only; the operator does not use them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn_peak.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// iters x 8 MFMAs of 16x16x32 per wave; the accumulators are summed and
// written once so that nothing is optimised away.
__global__ __launch_bounds__(256) void k_mfma_bf16(float* out, int iters, float seed) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(lane + e));
    b[e] = (__bf16)(seed * (float)(lane - e));
  }
  f32x4 c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i], 0, 0, 0);
  }
  f32x4 s = c[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) s += c[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

// dst[i] = src[i] over n 16-byte pieces
__global__ __launch_bounds__(256) void k_copy(const i32x4* __restrict__ src, i32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const i32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// one xor-sum per thread of n 16-byte pieces (written, so the reads stay)
__global__ __launch_bounds__(256) void k_read(const i32x4* __restrict__ src, size_t n, int* out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  i32x4 acc = i32x4{0, 0, 0, 0};
  for (; i + 3 * stride < n; i += 4 * stride) {
    const i32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n; i += stride) acc ^= src[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Wave 0 of one workgroup, iters rounds of: MODE 0, 32 reads of 1 KiB from
// LDS (ds_read_b128, 64 lanes x 16 contiguous bytes); MODE 1, the same reads
// each followed by one v_mfma_f32_16x16x32_bf16; MODE 2, the 32 MFMAs alone.
// The MFMAs accumulate into four independent chains.  The order is pinned
// with scheduling barriers (left alone, the compiler issues every read first
// and every MFMA after them), and each round ends by waiting for its reads;
// the read values are then only passed to an empty asm, so no vector ALU work
// on them is timed.  cycles[0] = the loop's shader-clock cycles.  A value
// that depends on the reads and the accumulators is written only if it
// matches a sentinel, so nothing is optimised away.
template <int MODE>
__global__ __launch_bounds__(256) void k_lds_wave(long long* cycles, int iters, int* sink) {
  constexpr int NR = MODE == 2 ? 0 : 32, NM = MODE == 0 ? 0 : 32;
  __shared__ __attribute__((aligned(1024))) char buf[32 * 1024];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 32 * 1024 / 4; i += blockDim.x) reinterpret_cast<int*>(buf)[i] = i;
  __syncthreads();
  if (w != 0) return;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(lane + e));
    b[e] = (__bf16)(2e-3f * (float)(lane - e));
  }
  f32x4 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  int acc = 0;
  const long long t0 = (long long)__builtin_readcyclecounter();
  for (int it = 0; it < iters; ++it) {
    i32x4 r[NR > 0 ? NR : 1];
#pragma unroll
    for (int i = 0; i < NR; ++i) r[i] = *reinterpret_cast<const i32x4*>(buf + i * 1024 + 16 * lane);
#pragma unroll
    for (int i = 0; i < NM; ++i) c[i & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i & 3], 0, 0, 0);
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      if (NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      if (NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NR; ++i) asm volatile("" ::"v"(r[i]));
    acc ^= NR ? r[0][0] : 0;
  }
  const long long t1 = (long long)__builtin_readcyclecounter();
  float f = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) f += c[i][0];
  if (lane == 0) cycles[0] = t1 - t0;
  if (acc == 0x13572468 || f == 12345.f) sink[lane] = acc;
}

}  // namespace

extern "C" {

int gdn_peak_lds_wave(long long* cycles, int* sink, int mode, int iters, void* stream) {
  if (!cycles || !sink || iters < 1 || mode < 0 || mode > 2) return (int)hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (mode == 0) hipLaunchKernelGGL(k_lds_wave<0>, dim3(1), dim3(256), 0, s, cycles, iters, sink);
  else if (mode == 1) hipLaunchKernelGGL(k_lds_wave<1>, dim3(1), dim3(256), 0, s, cycles, iters, sink);
  else hipLaunchKernelGGL(k_lds_wave<2>, dim3(1), dim3(256), 0, s, cycles, iters, sink);
  return (int)hipGetLastError();
}

int gdn_peak_mfma_bf16(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mfma_bf16, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), out, iters, 1e-3f);
  return (int)hipGetLastError();
}

int gdn_peak_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes % 16 || blocks < 1 || ((uintptr_t)src | (uintptr_t)dst) % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const i32x4*>(src), reinterpret_cast<i32x4*>(dst), bytes / 16);
  return (int)hipGetLastError();
}

int gdn_peak_read(const void* src, size_t bytes, int* out, int blocks, void* stream) {
  if (!src || !out || bytes % 16 || blocks < 1 || ((uintptr_t)src) % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const i32x4*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
