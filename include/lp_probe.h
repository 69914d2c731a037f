/*
 * lp_probe.h -- measurement helper shipped beside liblp.so as liblp_probe.so.
 *
 * Not an entry point of the log-prob path: bench.py uses it to measure the
 * HBM read bandwidth, the bf16 matrix-core rate and the v_exp_f32 rate the
 * GPU it runs on reaches, reported next to the datasheet peaks as second
 * denominators (and, for the exponential, the ALU budget of the row kernels,
 * which evaluate one per logit).
 */
#pragma once

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launches one streaming read of `bytes` bytes at device pointer `buf`
 * (16-byte aligned, bytes a positive multiple of 16) with `blocks`
 * workgroups of 256 threads, each reading one contiguous slice of
 * ceil(bytes / 16 / blocks) 16-byte words, on `stream` (a hipStream_t,
 * NULL = default).
 * `sink` is a device unsigned int the kernel may write (it does only when
 * the XOR of all words equals 0x9e3779b9); the caller owns both buffers.
 * Returns 0 on launch, 1 on an invalid argument (nothing launched), 2 if the
 * launch failed.  Asynchronous: time it with events on `stream`.
 */
int lp_probe_read(const void* buf, int64_t bytes, int blocks, unsigned* sink, void* stream);

/*
 * Launches `blocks` workgroups of 512 threads (8 waves, two per SIMD of a
 * CU), each wave issuing `iters` x 8 independent v_mfma_f32_32x32x16_bf16
 * (32768 flop each) from registers, on `stream`: total flop =
 * blocks x 8 x iters x 8 x 32768.  Thread 0 of workgroup b writes
 * clocks[4b .. 4b+3] = shader-clock counter before and after, fixed-frequency
 * counter before and after (the ratio of the two deltas times the
 * fixed counter's rate is the clock the workgroup ran at).  `clocks` is
 * device memory of 4 x blocks unsigned 64-bit words (8-byte aligned), `sink`
 * a device float the kernel writes only if its accumulators sum to a marker.
 * Returns 0 on launch, 1 on an invalid argument (nothing launched), 2 if the
 * launch failed.
 */
int lp_probe_mfma(int blocks, int iters, unsigned long long* clocks, float* sink, void* stream);

/*
 * Launches `blocks` workgroups of 1024 threads (16 waves, four per SIMD),
 * each lane running `iters` x 16 v_exp_f32 (sixteen independent chains
 * x <- 2^-x, no other arithmetic), on `stream`: total exp2 evaluations =
 * blocks x 1024 x iters x 16.
 * `clocks` and `sink` as for lp_probe_mfma (same clock records, same
 * ownership).  Returns 0 on launch, 1 on an invalid argument (nothing
 * launched), 2 if the launch failed.
 */
int lp_probe_exp(int blocks, int iters, unsigned long long* clocks, float* sink, void* stream);

/*
 * Host query of the current device: the rate of the fixed-frequency counter
 * that lp_probe_mfma reads (kHz) and the peak shader clock (kHz).  Returns 0,
 * 1 for NULL arguments, 2 if the runtime query failed.
 */
int lp_probe_clock_rates(int* wall_khz, int* peak_khz);

#ifdef __cplusplus
}
#endif
