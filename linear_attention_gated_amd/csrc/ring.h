// ring.h -- LDS ring buffer fed by direct global->LDS loads (gfx950).
//
// The sequential state passes walk the chunks of a sequence one after the
// other; every chunk's operands are known in advance (they do not depend on
// the state), so they are streamed into a ring of S LDS slots ahead of use.
// A workgroup has one compute wave and S-1 loader waves.  Loader l fills the
// chunks c with c % (S-1) == l, one chunk at a time, with
// global_load_lds_dwordx4 (64 lanes x 16 bytes per instruction, written to
// LDS contiguously, so fragment-native records land as they are stored).
// One workgroup barrier per chunk orders the ring:
//   step c:  loader of chunk c waits for its loads (vmcnt(0)); barrier;
//            compute wave reads slot c % S;
//            loader of chunk c refills slot (c-1) % S with chunk c + S - 1.
// Each loader has at most one chunk in flight, which keeps its vmcnt well
// inside the hardware limit, and the ring runs S-1 chunks ahead.  The
// barrier is the bare s_barrier: no wave waits for its own global stores.
#pragma once
#include "frag.h"

namespace gdn {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// One wave copies `bytes` (a multiple of 1024) from global memory to LDS.
__device__ __forceinline__ void dma_kib(const void* src, void* dst, int bytes, int lane) {
  const char* s = reinterpret_cast<const char*>(src);
  char* d = reinterpret_cast<char*>(dst);
  for (int off = 0; off < bytes; off += 1024)
    __builtin_amdgcn_global_load_lds(s + off + 16 * lane, (lds_void_ptr)(d + off), 16, 0, 0);
}

// As dma_kib, with the 1 KiB pieces taken in rotated order from piece `rot`
// (0 <= rot): the same bytes, a different first address.
__device__ __forceinline__ void dma_kib_rot(const void* src, void* dst, int bytes, int lane, int rot) {
  const char* s = reinterpret_cast<const char*>(src);
  char* d = reinterpret_cast<char*>(dst);
  const int n = bytes / 1024;
  for (int i = 0; i < n; ++i) {
    const int off = ((i + rot) % n) * 1024;
    __builtin_amdgcn_global_load_lds(s + off + 16 * lane, (lds_void_ptr)(d + off), 16, 0, 0);
  }
}

// One wave copies 256 bytes (64 lanes x 4 bytes).
__device__ __forceinline__ void dma_256(const void* src, void* dst, int lane) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src) + 4 * lane, (lds_void_ptr)dst, 4, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Number of slots that fit in the 160 KiB of LDS, between 2 and 4.
constexpr int ring_slots(int slot_bytes) {
  return (160 * 1024 / slot_bytes) >= 4 ? 4 : ((160 * 1024 / slot_bytes) >= 3 ? 3 : 2);
}

}  // namespace gdn
