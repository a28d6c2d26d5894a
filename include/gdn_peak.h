/*
 * gdn_peak.h -- C ABI of libgdn_peak.so: microbenchmarks that measure the
 * peaks of the GPU the operator runs on (AMD MI355X, gfx950), so that each
 * kernel's achieved rate can be read against a measured ceiling as well as the
 * published one.  Diagnostics only: nothing here is part of the operator.
 *
 * All pointers are device pointers owned by the caller; work is enqueued on
 * `stream` (hipStream_t as void*, NULL = the null stream) and the calls return
 * without waiting.  Each returns 0 (hipSuccess) or a hipError_t code; invalid
 * arguments return hipErrorInvalidValue before anything is launched.
 */
#ifndef GDN_PEAK_H_
#define GDN_PEAK_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 matrix-core rate: `blocks` workgroups of 256 threads (4 waves),
 * each wave issuing iters x 8 v_mfma_f32_16x16x32_bf16 (16,384 flops each) on
 * independent accumulators.  out: blocks * 256 floats, written. */
int gdn_peak_mfma_bf16(float* out, int blocks, int iters, void* stream);

/* HBM copy: dst = src over `bytes` (a multiple of 16; both 16-byte aligned,
 * not overlapping), `blocks` workgroups of 256 threads. */
int gdn_peak_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);

/* HBM read: every 16-byte piece of src is read once; out: blocks * 256 ints,
 * written (an xor of the data, so the reads cannot be dropped). */
int gdn_peak_read(const void* src, size_t bytes, int* out, int blocks, void* stream);

/* One wave's LDS reads and MFMAs: wave 0 of one workgroup runs iters rounds of
 * mode 0: 32 reads of 1 KiB from LDS with ds_read_b128 (64 lanes x 16
 * contiguous bytes), waited for at the round's end; mode 1: the same reads,
 * each followed by one v_mfma_f32_16x16x32_bf16 (order pinned); mode 2: the 32
 * MFMAs alone (four independent accumulator chains in modes 1 and 2).
 * cycles[0] (one long long, device) receives the loop's shader-clock cycles:
 * cycles[0] / (32 iters) is the cost to that wave of one read, one read with
 * one MFMA, or one MFMA.  sink: 64 ints, written only if the data matches a
 * sentinel (keeps the work).  Invalid pointers, iters < 1 or a mode outside
 * 0..2 return hipErrorInvalidValue. */
int gdn_peak_lds_wave(long long* cycles, int* sink, int mode, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PEAK_H_ */
