/*
 * lp_probe.h -- measurement helper shipped beside liblp.so as liblp_probe.so.
 *
 * Not an entry point of the log-prob path: bench.py uses it to measure the
 * HBM read bandwidth the GPU it runs on reaches, reported next to the
 * datasheet peak as a second denominator for the HBM-bound kernels.
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

#ifdef __cplusplus
}
#endif
