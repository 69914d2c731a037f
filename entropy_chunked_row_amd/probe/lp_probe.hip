// Measurement helpers (not part of the log-prob path), so that bench.py can
// report what this GPU actually reaches next to the datasheet figures:
//   k_probe_read   a streaming read of a device buffer.  Each workgroup reads
//                  one contiguous slice (the pattern of the row kernels, one
//                  row per workgroup); each thread keeps U 16-byte
//                  non-temporal loads in flight and folds them into one value
//                  that is stored only if it equals a marker (never, for the
//                  caller's fill), which keeps the loads alive.
//   k_probe_mfma   back-to-back v_mfma_f32_32x32x16_bf16 from registers, two
//                  waves per SIMD, eight independent accumulators per wave;
//                  each workgroup also reads the shader-clock counter and the
//                  fixed-frequency counter at its start and end, which gives
//                  the clock the matrix cores ran at.
//   k_probe_exp    back-to-back v_exp_f32 (the transcendental unit that the
//                  row kernels use once per logit), same clock records.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lp_probe.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int U>
__global__ void __launch_bounds__(256) k_probe_read(const u32x4_t* __restrict__ p, int64_t n, int64_t per_block,
                                                    unsigned* out) {
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per_block;
  const int64_t e = b0 + per_block < n ? b0 + per_block : n;
  unsigned acc = 0;
  int64_t i = b0 + threadIdx.x;
  for (; i + (U - 1) * 256 < e; i += U * 256) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < e; i += 256) {
    const u32x4_t v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) out[0] = acc;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 8 waves (two per SIMD); per iteration each wave issues one MFMA into each
// of its 8 accumulators, so consecutive MFMAs of a wave never depend on each
// other.  Thread 0 records (shader clock, fixed clock) before the loop and
// after every wave of the workgroup has finished; the accumulators feed one
// value stored only if it equals a marker, which keeps the MFMAs alive.
__global__ void __launch_bounds__(512) k_probe_mfma(int iters, unsigned long long* __restrict__ clocks,
                                                    float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(static_cast<float>(lane + i) * (1.0f / 1024.0f));
    b[i] = static_cast<__bf16>(static_cast<float>(lane - i) * (1.0f / 2048.0f));
  }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  __syncthreads();
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
  __syncthreads();  // every wave's MFMAs are done
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
  if (s == 1234.5f) sink[0] = s;
}

// 16 waves per workgroup (four per SIMD: the exponential's latency needs
// that many waves in flight to reach its issue rate); each lane runs 16
// independent chains x <- 2^(-x) (one v_exp_f32 with a negated source per
// step, no other arithmetic; the chains stay in (0.5, 1]).  Thread 0 records
// the same clock pairs as k_probe_mfma.
__global__ void __launch_bounds__(1024) k_probe_exp(int iters, unsigned long long* __restrict__ clocks,
                                                    float* __restrict__ sink) {
  float x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = 0.5f + static_cast<float>((threadIdx.x + j) & 63) * (1.0f / 128.0f);
  __syncthreads();
  unsigned long long t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += x[j];
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    clocks[4 * blockIdx.x + 0] = t0;
    clocks[4 * blockIdx.x + 1] = t1;
    clocks[4 * blockIdx.x + 2] = r0;
    clocks[4 * blockIdx.x + 3] = r1;
  }
  if (s == 1234.5f) sink[0] = s;
}

}  // namespace

extern "C" int lp_probe_exp(int blocks, int iters, unsigned long long* clocks, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || !clocks || !sink) return 1;
  if ((reinterpret_cast<uintptr_t>(clocks) & 7u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return 1;
  hipLaunchKernelGGL(k_probe_exp, dim3(static_cast<unsigned>(blocks)), dim3(1024), 0, static_cast<hipStream_t>(stream),
                     iters, clocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int lp_probe_mfma(int blocks, int iters, unsigned long long* clocks, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || !clocks || !sink) return 1;
  if ((reinterpret_cast<uintptr_t>(clocks) & 7u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return 1;
  hipLaunchKernelGGL(k_probe_mfma, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, static_cast<hipStream_t>(stream),
                     iters, clocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int lp_probe_read(const void* buf, int64_t bytes, int blocks, unsigned* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || blocks <= 0) return 1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return 1;
  const int64_t n = bytes / 16;
  const int64_t per_block = (n + blocks - 1) / blocks;
  hipLaunchKernelGGL(k_probe_read<8>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(buf), n, per_block, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int lp_probe_clock_rates(int* wall_khz, int* peak_khz) {
  if (!wall_khz || !peak_khz) return 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 2;
  if (hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 2;
  if (hipDeviceGetAttribute(peak_khz, hipDeviceAttributeClockRate, dev) != hipSuccess) return 2;
  return 0;
}
