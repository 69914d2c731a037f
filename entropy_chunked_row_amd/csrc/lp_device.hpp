// Device-side building blocks shared by the row-reduction kernels and the
// fused LM-head epilogues.
//
// Row state.  For one row (or any subset of its vocabulary) the kernels keep
//   mc = RN(max_z * c)            reference exponent, log2 units
//   s  = sum_j 2^{t_j}            t_j = RN(z_j * c - mc)
//   a  = sum_j 2^{t_j} * t_j
// with c = log2(e) / tau (tau = 1 when the temperature does not apply).  Then
//   log-sum-exp of z / tau = ln2 * (mc + log2 s)
//   log p(y)               = ln2 * (t_y - log2 s)
//   entropy                = ln2 * (log2 s - a / s)
// Two states over disjoint parts of a row merge exactly (up to rounding) by
// moving both to the larger reference exponent.  Every sum is fp32; the
// model-precision values are only ever widened, never accumulated in place.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309417f;
// Reference exponent of a state that has seen nothing.  Finite on purpose: a
// -inf element then gives t = -inf (probability 0) instead of NaN.
constexpr float kNegBig = -3.402823466e38f;

struct Stat {
  float mc, s, a;
};

__device__ __forceinline__ Stat stat_empty() { return Stat{kNegBig, 0.f, 0.f}; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge two partial states of the same row.
__device__ __forceinline__ Stat stat_merge(Stat x, Stat y) {
  const float mc = fmaxf(x.mc, y.mc);
  float s = 0.f, a = 0.f;
  if (x.s > 0.f) {
    const float d = x.mc - mc;
    const float r = fast_exp2(d);
    s += x.s * r;
    a += (x.a + x.s * d) * r;
  }
  if (y.s > 0.f) {
    const float d = y.mc - mc;
    const float r = fast_exp2(d);
    s += y.s * r;
    a += (y.a + y.s * d) * r;
  }
  return Stat{mc, s, a};
}

// Move a state to a new, larger reference exponent nmc.
__device__ __forceinline__ void stat_rebase(Stat& st, float nmc) {
  if (st.s > 0.f) {
    const float d = st.mc - nmc;
    const float r = fast_exp2(d);
    st.a = (st.a + st.s * d) * r;
    st.s *= r;
  }
  st.mc = nmc;
}

// Fold N widened values into the state: one max test, then CH-long partial
// sums (short chains keep fp32 rounding low).  GUARD clamps t so that a -inf
// value contributes 0 * finite instead of 0 * -inf to `a`.
template <bool GUARD, int N, int CH>
__device__ __forceinline__ void stat_push(Stat& st, const float* x, float c) {
  float vm = x[0];
#pragma unroll
  for (int k = 1; k < N; ++k) vm = fmaxf(vm, x[k]);
  const float vmc = vm * c;
  if (vmc > st.mc) stat_rebase(st, vmc);
  const float nmc = -st.mc;
#pragma unroll
  for (int g = 0; g < N; g += CH) {
    float ps = 0.f, pa = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      float t = fmaf(x[g + k], c, nmc);
      if (GUARD) t = fmaxf(t, kNegBig);
      const float e = fast_exp2(t);
      ps += e;
      pa = fmaf(e, t, pa);
    }
    st.s += ps;
    st.a += pa;
  }
}

// Butterfly over a wave64: every lane ends with the merge of all 64 lanes.
__device__ __forceinline__ Stat stat_wave_allreduce(Stat st) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Stat o;
    o.mc = __shfl_xor(st.mc, off, 64);
    o.s = __shfl_xor(st.s, off, 64);
    o.a = __shfl_xor(st.a, off, 64);
    st = stat_merge(st, o);
  }
  return st;
}

// Block-wide merge; every thread returns the same state (fixed order, so the
// result is bitwise reproducible).  `sm` holds NT/64 states.
template <int NT>
__device__ __forceinline__ Stat stat_block_allreduce(Stat st, Stat* sm) {
  constexpr int NW = NT / 64;
  st = stat_wave_allreduce(st);
  if (NW == 1) return st;
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm[w] = st;
  __syncthreads();
  Stat r = sm[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) r = stat_merge(r, sm[k]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// element types: 16-byte vectors and exact widening to fp32
// ---------------------------------------------------------------------------

struct Bf16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ void unpack(u32x4 w, float* x) {
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
    x[4] = __uint_as_float(w.z << 16);
    x[5] = __uint_as_float(w.z & 0xffff0000u);
    x[6] = __uint_as_float(w.w << 16);
    x[7] = __uint_as_float(w.w & 0xffff0000u);
  }
  __device__ static __forceinline__ float load1(const char* p, int64_t i) {
    const uint16_t b = reinterpret_cast<const uint16_t*>(p)[i];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  }
};

__device__ __forceinline__ float half_bits_to_float(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

struct Fp16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ void unpack(u32x4 w, float* x) {
    x[0] = half_bits_to_float(w.x & 0xffffu);
    x[1] = half_bits_to_float(w.x >> 16);
    x[2] = half_bits_to_float(w.y & 0xffffu);
    x[3] = half_bits_to_float(w.y >> 16);
    x[4] = half_bits_to_float(w.z & 0xffffu);
    x[5] = half_bits_to_float(w.z >> 16);
    x[6] = half_bits_to_float(w.w & 0xffffu);
    x[7] = half_bits_to_float(w.w >> 16);
  }
  __device__ static __forceinline__ float load1(const char* p, int64_t i) {
    return half_bits_to_float(reinterpret_cast<const uint16_t*>(p)[i]);
  }
};

struct Fp32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  __device__ static __forceinline__ void unpack(u32x4 w, float* x) {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
  __device__ static __forceinline__ float load1(const char* p, int64_t i) {
    return reinterpret_cast<const float*>(p)[i];
  }
};

// Dual (student u, teacher v) state for KL(teacher || student).
// Student u: (mcu, su).  Teacher v: (mcv, sv) and C = sum_j 2^{tv_j} (v_j - u_j)
// on the teacher's reference.  Then, with natural-log normalisers
// lse = ln2 (mc + log2 s):  KL = C / sv - (lse_v - lse_u).

struct KLState {
  float mcu, su, mcv, sv, C;
};

template <bool GUARD, int N, int CH>
__device__ __forceinline__ void kl_push(KLState& st, const float* xu, const float* xv, float c) {
  float mu = xu[0], mv = xv[0];
#pragma unroll
  for (int k = 1; k < N; ++k) {
    mu = fmaxf(mu, xu[k]);
    mv = fmaxf(mv, xv[k]);
  }
  const float muc = mu * c, mvc = mv * c;
  if (muc > st.mcu) {
    if (st.su > 0.f) st.su *= fast_exp2(st.mcu - muc);
    st.mcu = muc;
  }
  if (mvc > st.mcv) {
    if (st.sv > 0.f) {
      const float r = fast_exp2(st.mcv - mvc);
      st.sv *= r;
      st.C *= r;
    }
    st.mcv = mvc;
  }
  const float nu = -st.mcu, nv = -st.mcv;
#pragma unroll
  for (int g = 0; g < N; g += CH) {
    float pu = 0.f, pv = 0.f, pc = 0.f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const float eu = fast_exp2(fmaf(xu[g + k], c, nu));
      const float ev = fast_exp2(fmaf(xv[g + k], c, nv));
      pu += eu;
      pv += ev;
      const float d = xv[g + k] - xu[g + k];
      if (GUARD)
        pc += (ev > 0.f) ? ev * d : 0.f;
      else
        pc = fmaf(ev, d, pc);
    }
    st.su += pu;
    st.sv += pv;
    st.C += pc;
  }
}

__device__ __forceinline__ KLState kl_merge(KLState x, KLState y) {
  KLState r;
  r.mcu = fmaxf(x.mcu, y.mcu);
  r.su = 0.f;
  if (x.su > 0.f) r.su += x.su * fast_exp2(x.mcu - r.mcu);
  if (y.su > 0.f) r.su += y.su * fast_exp2(y.mcu - r.mcu);
  r.mcv = fmaxf(x.mcv, y.mcv);
  r.sv = 0.f;
  r.C = 0.f;
  if (x.sv > 0.f) {
    const float f = fast_exp2(x.mcv - r.mcv);
    r.sv += x.sv * f;
    r.C += x.C * f;
  }
  if (y.sv > 0.f) {
    const float f = fast_exp2(y.mcv - r.mcv);
    r.sv += y.sv * f;
    r.C += y.C * f;
  }
  return r;
}

// Split of a row of `n` elements at `p` into a scalar head (up to the first
// 16-byte boundary), whole 16-byte vectors, and a scalar tail.
template <class Tr>
struct RowSplit {
  int head;
  int nvec;
  int tail;
  __device__ __forceinline__ RowSplit(const char* p, int n) {
    const int mis = static_cast<int>(reinterpret_cast<uintptr_t>(p) & 15u);
    int hd = mis ? (16 - mis) / Tr::kBytes : 0;
    head = hd < n ? hd : n;
    nvec = (n - head) / Tr::kPerVec;
    tail = n - head - nvec * Tr::kPerVec;
  }
};

}  // namespace lp
