// Memory-bound row reductions over model-precision logits:
//   * k_logprobs_entropy: log p(target) and entropy per scored row
//     (miles PR #2764 summary, "关键源码片段": chunked upcast to fp32, then the
//     temperature divide in fp32, then the log-softmax at the target).
//   * k_kl_full_vocab: exact KL(teacher || student) per row plus both target
//     log-probs and the masked |exp(a) - exp(b)| (DeepSeek-V4 book ch.19,
//     "TileLang KL Kernel"; msprobe probs_diff page §3.2).
//   * k_prob_diff: the same diff on two given log-prob arrays.
//
// One workgroup per row.  Each lane streams 16-byte vectors (8 bf16/fp16 or
// 4 fp32) with non-temporal loads, U vectors in flight, widens them in
// registers and folds them into its running (mc, s, a) state; the workgroup
// then merges the lane states.  Nothing but the per-row outputs is written.
#include "lp_device.hpp"
#include "lp_internal.hpp"

namespace lp {

// ---------------------------------------------------------------------------
// logits-input log-prob + entropy
// ---------------------------------------------------------------------------

template <class Tr, int NT, int U, bool GUARD>
__device__ __forceinline__ Stat scan_row(const char* rowp, const RowSplit<Tr>& sp, float c) {
  constexpr int P = Tr::kPerVec;
  const int tid = threadIdx.x;
  Stat st = stat_empty();
  if (tid < sp.head) {
    float x = Tr::load1(rowp, tid);
    stat_push<GUARD, 1, 1>(st, &x, c);
  }
  const u32x4* vp = reinterpret_cast<const u32x4*>(rowp + sp.head * Tr::kBytes);
  int i = tid;
  for (; i + (U - 1) * NT < sp.nvec; i += U * NT) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = __builtin_nontemporal_load(vp + i + u * NT);
    float x[U * P];
#pragma unroll
    for (int u = 0; u < U; ++u) Tr::unpack(w[u], x + u * P);
    stat_push<GUARD, U * P, P>(st, x, c);
  }
  for (; i < sp.nvec; i += NT) {
    const u32x4 w = __builtin_nontemporal_load(vp + i);
    float x[P];
    Tr::unpack(w, x);
    stat_push<GUARD, P, P>(st, x, c);
  }
  if (tid < sp.tail) {
    float x = Tr::load1(rowp, sp.head + sp.nvec * P + tid);
    stat_push<GUARD, 1, 1>(st, &x, c);
  }
  return st;
}

template <class Tr, int NT, int U>
__global__ void __launch_bounds__(NT) k_logprobs_entropy(RowArgs args) {
  __shared__ Stat sm[NT / 64];
  const int64_t row = args.row0 + blockIdx.x;
  if (args.mask && args.mask[row] == 0) {
    for (int k = threadIdx.x; k < args.K; k += NT) args.logprob[row * args.K + k] = 0.f;
    if (threadIdx.x == 0 && args.entropy) args.entropy[row] = 0.f;
    return;
  }
  const char* rowp = static_cast<const char*>(args.x) + row * args.ld * Tr::kBytes;
  const int V = args.V;
  const RowSplit<Tr> sp(rowp, V);
  const float c = args.c;
  Stat st = stat_block_allreduce<NT>(scan_row<Tr, NT, U, false>(rowp, sp, c), sm);
  // A -inf logit makes `a` NaN (0 * -inf) while `s` stays finite: redo the
  // row with the clamped fold.  Every thread holds the same merged state, so
  // the branch is uniform.
  if (__builtin_isnan(st.a) && !__builtin_isnan(st.s))
    st = stat_block_allreduce<NT>(scan_row<Tr, NT, U, true>(rowp, sp, c), sm);
  const float l2s = log2f(st.s);
  for (int k = threadIdx.x; k < args.K; k += NT) {
    const int64_t y = args.targets[row * args.K + k];
    float lp = __builtin_nanf("");
    if (y >= 0 && y < V) {
      const float ty = fmaf(Tr::load1(rowp, y), c, -st.mc);
      lp = (ty - l2s) * kLn2;
    }
    args.logprob[row * args.K + k] = lp;
  }
  if (threadIdx.x == 0 && args.entropy) args.entropy[row] = (l2s - st.a / st.s) * kLn2;
}

// Workgroup size and 16-byte loads in flight per lane for rows longer than
// 16384 (build-time knobs; measured defaults).
#ifndef LP_ROWS_NT
#define LP_ROWS_NT 256
#endif
#ifndef LP_ROWS_U
#define LP_ROWS_U 8
#endif

// Rows per launch of the one-row-per-workgroup kernels: keeps a dispatch far
// below 2^32 work-items for any row count.
constexpr int64_t kRowsPerLaunch = int64_t(1) << 22;

template <class Tr>
static hipError_t launch_rows_t(const RowArgs& a, hipStream_t s) {
  for (int64_t r0 = 0; r0 < a.rows; r0 += kRowsPerLaunch) {
    RowArgs b = a;
    b.row0 = a.row0 + r0;
    b.rows = a.rows - r0 < kRowsPerLaunch ? a.rows - r0 : kRowsPerLaunch;
    const unsigned grid = static_cast<unsigned>(b.rows);
    TimedLaunch tl("k_logprobs_entropy", s);
    if (b.V <= 2048) {
      hipLaunchKernelGGL((k_logprobs_entropy<Tr, 64, 2>), dim3(grid), dim3(64), 0, s, b);
    } else if (b.V <= 16384) {
      hipLaunchKernelGGL((k_logprobs_entropy<Tr, 128, 4>), dim3(grid), dim3(128), 0, s, b);
    } else {
      hipLaunchKernelGGL((k_logprobs_entropy<Tr, LP_ROWS_NT, LP_ROWS_U>), dim3(grid), dim3(LP_ROWS_NT), 0, s, b);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_logprobs_entropy(int dtype, const RowArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  switch (dtype) {
    case 0: return launch_rows_t<Bf16>(a, s);
    case 1: return launch_rows_t<Fp16>(a, s);
    default: return launch_rows_t<Fp32>(a, s);
  }
}

// ---------------------------------------------------------------------------
// exact KL(teacher || student) over the full vocabulary
// ---------------------------------------------------------------------------
// The dual state (KLState, kl_push, kl_merge) is shared with the fused LM-head
// KL and lives with the other device helpers.

template <int NT>
__device__ __forceinline__ KLState kl_block_allreduce(KLState st, KLState* sm) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    KLState o;
    o.mcu = __shfl_xor(st.mcu, off, 64);
    o.su = __shfl_xor(st.su, off, 64);
    o.mcv = __shfl_xor(st.mcv, off, 64);
    o.sv = __shfl_xor(st.sv, off, 64);
    o.C = __shfl_xor(st.C, off, 64);
    st = kl_merge(st, o);
  }
  constexpr int NW = NT / 64;
  if (NW == 1) return st;
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sm[w] = st;
  __syncthreads();
  KLState r = sm[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) r = kl_merge(r, sm[k]);
  __syncthreads();
  return r;
}

template <class Tr, int NT, int U, bool GUARD>
__device__ __forceinline__ KLState scan_kl(const char* up, const char* vp, int V, bool aligned_pair, float c) {
  constexpr int P = Tr::kPerVec;
  const int tid = threadIdx.x;
  KLState st{kNegBig, 0.f, kNegBig, 0.f, 0.f};
  if (aligned_pair) {
    // both rows share the same 16-byte phase
    const RowSplit<Tr> sp(up, V);
    for (int j = tid; j < sp.head; j += NT) {
      float xu = Tr::load1(up, j), xv = Tr::load1(vp, j);
      kl_push<GUARD, 1, 1>(st, &xu, &xv, c);
    }
    const u32x4* uq = reinterpret_cast<const u32x4*>(up + sp.head * Tr::kBytes);
    const u32x4* vq = reinterpret_cast<const u32x4*>(vp + sp.head * Tr::kBytes);
    int i = tid;
    for (; i + (U - 1) * NT < sp.nvec; i += U * NT) {
      u32x4 wu[U], wv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        wu[u] = __builtin_nontemporal_load(uq + i + u * NT);
        wv[u] = __builtin_nontemporal_load(vq + i + u * NT);
      }
      float xu[U * P], xv[U * P];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        Tr::unpack(wu[u], xu + u * P);
        Tr::unpack(wv[u], xv + u * P);
      }
      kl_push<GUARD, U * P, P>(st, xu, xv, c);
    }
    for (; i < sp.nvec; i += NT) {
      float xu[P], xv[P];
      Tr::unpack(__builtin_nontemporal_load(uq + i), xu);
      Tr::unpack(__builtin_nontemporal_load(vq + i), xv);
      kl_push<GUARD, P, P>(st, xu, xv, c);
    }
    const int t0 = sp.head + sp.nvec * P;
    for (int j = t0 + tid; j < V; j += NT) {
      float xu = Tr::load1(up, j), xv = Tr::load1(vp, j);
      kl_push<GUARD, 1, 1>(st, &xu, &xv, c);
    }
  } else {
    for (int j = tid; j < V; j += NT) {
      float xu = Tr::load1(up, j), xv = Tr::load1(vp, j);
      kl_push<GUARD, 1, 1>(st, &xu, &xv, c);
    }
  }
  return st;
}

template <class Tr, int NT, int U>
__global__ void __launch_bounds__(NT) k_kl_full_vocab(KLArgs args) {
  __shared__ KLState sm[NT / 64];
  const int64_t row = args.row0 + blockIdx.x;
  const char* up = static_cast<const char*>(args.student) + row * args.ld_s * Tr::kBytes;
  const char* vp = static_cast<const char*>(args.teacher) + row * args.ld_t * Tr::kBytes;
  const int V = args.V;
  const bool aligned_pair = ((reinterpret_cast<uintptr_t>(up) ^ reinterpret_cast<uintptr_t>(vp)) & 15u) == 0;
  const float c = args.c;
  KLState st = kl_block_allreduce<NT>(scan_kl<Tr, NT, U, false>(up, vp, V, aligned_pair, c), sm);
  if (__builtin_isnan(st.C) && !__builtin_isnan(st.su) && !__builtin_isnan(st.sv))
    st = kl_block_allreduce<NT>(scan_kl<Tr, NT, U, true>(up, vp, V, aligned_pair, c), sm);
  if (threadIdx.x == 0) {
    const float l2u = log2f(st.su), l2v = log2f(st.sv);
    const float dlse = ((st.mcv - st.mcu) + (l2v - l2u)) * kLn2;
    args.kl[row] = st.C / st.sv - dlse;
    if (args.targets) {
      const int64_t y = args.targets[row];
      float lpu = __builtin_nanf(""), lpv = __builtin_nanf("");
      if (y >= 0 && y < V) {
        lpu = (fmaf(Tr::load1(up, y), c, -st.mcu) - l2u) * kLn2;
        lpv = (fmaf(Tr::load1(vp, y), c, -st.mcv) - l2v) * kLn2;
      }
      if (args.lp_student) args.lp_student[row] = lpu;
      if (args.lp_teacher) args.lp_teacher[row] = lpv;
      if (args.prob_diff) {
        const bool keep = args.diff_mask == nullptr || args.diff_mask[row] != 0;
        args.prob_diff[row] = keep ? fabsf(expf(lpu) - expf(lpv)) : 0.f;
      }
    }
  }
}

// 16-byte loads in flight per lane and per row (student and teacher each)
// for rows longer than 2048 (build-time knob; measured default).
#ifndef LP_KL_ROWS_U
#define LP_KL_ROWS_U 4
#endif

template <class Tr>
static hipError_t launch_kl_t(const KLArgs& a, hipStream_t s) {
  for (int64_t r0 = 0; r0 < a.T; r0 += kRowsPerLaunch) {
    KLArgs b = a;
    b.row0 = r0;
    const unsigned grid = static_cast<unsigned>(a.T - r0 < kRowsPerLaunch ? a.T - r0 : kRowsPerLaunch);
    TimedLaunch tl("k_kl_full_vocab", s);
    if (b.V <= 2048) {
      hipLaunchKernelGGL((k_kl_full_vocab<Tr, 64, 2>), dim3(grid), dim3(64), 0, s, b);
    } else {
      hipLaunchKernelGGL((k_kl_full_vocab<Tr, 256, LP_KL_ROWS_U>), dim3(grid), dim3(256), 0, s, b);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_kl_full_vocab(int dtype, const KLArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  switch (dtype) {
    case 0: return launch_kl_t<Bf16>(a, s);
    case 1: return launch_kl_t<Fp16>(a, s);
    default: return launch_kl_t<Fp32>(a, s);
  }
}

// ---------------------------------------------------------------------------
// elementwise prob diff
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) k_prob_diff(const float* __restrict__ a, const float* __restrict__ b,
                                                   const uint8_t* __restrict__ mask, int64_t n,
                                                   float* __restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const bool keep = mask == nullptr || mask[i] != 0;
    out[i] = keep ? fabsf(expf(a[i]) - expf(b[i])) : 0.f;
  }
}

hipError_t launch_prob_diff(const float* a, const float* b, const uint8_t* mask, int64_t n, float* out,
                            hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  TimedLaunch tl("k_prob_diff", s);
  hipLaunchKernelGGL(k_prob_diff, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a, b, mask, n, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// aggregates of the masked prob diff (two deterministic passes, fp64)
// ---------------------------------------------------------------------------
// Each thread sums its strided positions shifted by the first value it kept
// (so a lone or constant series has exactly zero spread), turns the sums into
// (count, mean, centred second moments), and the partials are combined with
// the pairwise update for means and co-moments (Chan, Golub and LeVeque) in a
// fixed order: the result is the same on every call.

constexpr int kStatsBlocks = 512;
constexpr int kStatsFields = 9;

size_t prob_diff_stats_workspace_bytes() { return sizeof(double) * kStatsBlocks * kStatsFields; }

// n, mean d, M2 d, max d, mean pa, mean pb, M2 pa, M2 pb, co-moment pa pb
struct Moments {
  double n, md, m2d, mx, ma, mb, m2a, m2b, cab;
};

__device__ inline Moments moments_merge(const Moments& x, const Moments& y) {
  if (y.n == 0.0) return x;
  if (x.n == 0.0) return y;
  Moments r;
  r.n = x.n + y.n;
  const double f = y.n / r.n, w = x.n * y.n / r.n;
  const double dd = y.md - x.md, da = y.ma - x.ma, db = y.mb - x.mb;
  r.md = x.md + dd * f;
  r.ma = x.ma + da * f;
  r.mb = x.mb + db * f;
  r.m2d = x.m2d + y.m2d + dd * dd * w;
  r.m2a = x.m2a + y.m2a + da * da * w;
  r.m2b = x.m2b + y.m2b + db * db * w;
  r.cab = x.cab + y.cab + da * db * w;
  r.mx = x.mx > y.mx ? x.mx : y.mx;
  return r;
}

__device__ inline void moments_store(double* p, const Moments& m) {
  p[0] = m.n; p[1] = m.md; p[2] = m.m2d; p[3] = m.mx; p[4] = m.ma;
  p[5] = m.mb; p[6] = m.m2a; p[7] = m.m2b; p[8] = m.cab;
}

__device__ inline Moments moments_load(const double* p) {
  return Moments{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8]};
}

__global__ void __launch_bounds__(256) k_prob_diff_stats_partial(const float* __restrict__ a,
                                                                 const float* __restrict__ b,
                                                                 const uint8_t* __restrict__ mask, int64_t n,
                                                                 double* __restrict__ part) {
  __shared__ double sm[256 * kStatsFields];
  double cnt = 0, kd = 0, ka = 0, kb = 0, sd = 0, sdd = 0, sa = 0, saa = 0, sb = 0, sbb = 0, sab = 0, mx = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (mask != nullptr && mask[i] == 0) continue;
    const double pa = exp(static_cast<double>(a[i]));
    const double pb = exp(static_cast<double>(b[i]));
    const double d = fabs(pa - pb);
    if (cnt == 0.0) {
      kd = d;
      ka = pa;
      kb = pb;
    }
    cnt += 1.0;
    const double xd = d - kd, xa = pa - ka, xb = pb - kb;
    sd += xd;
    sdd += xd * xd;
    sa += xa;
    saa += xa * xa;
    sb += xb;
    sbb += xb * xb;
    sab += xa * xb;
    mx = d > mx ? d : mx;
  }
  Moments m{0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (cnt > 0.0) {
    m.n = cnt;
    m.md = kd + sd / cnt;
    m.ma = ka + sa / cnt;
    m.mb = kb + sb / cnt;
    m.m2d = fmax(sdd - sd * sd / cnt, 0.0);
    m.m2a = fmax(saa - sa * sa / cnt, 0.0);
    m.m2b = fmax(sbb - sb * sb / cnt, 0.0);
    m.cab = sab - sa * sb / cnt;
    m.mx = mx;
  }
  moments_store(sm + threadIdx.x * kStatsFields, m);
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      const Moments x = moments_load(sm + threadIdx.x * kStatsFields);
      const Moments y = moments_load(sm + (threadIdx.x + off) * kStatsFields);
      moments_store(sm + threadIdx.x * kStatsFields, moments_merge(x, y));
    }
    __syncthreads();
  }
  if (threadIdx.x < kStatsFields) part[blockIdx.x * kStatsFields + threadIdx.x] = sm[threadIdx.x];
}

__global__ void __launch_bounds__(64) k_prob_diff_stats_final(const double* __restrict__ part, int nblocks,
                                                              double* __restrict__ out) {
  if (threadIdx.x != 0) return;
  Moments m{0, 0, 0, 0, 0, 0, 0, 0, 0};
  for (int bl = 0; bl < nblocks; ++bl) m = moments_merge(m, moments_load(part + bl * kStatsFields));
  if (m.n == 0.0) {
    out[0] = 0.0;
    out[1] = 0.0;
    out[2] = 0.0;
    out[3] = 0.0;
    out[4] = __builtin_nan("");
    return;
  }
  out[0] = m.n;
  out[1] = m.mx;
  out[2] = m.md;
  out[3] = sqrt(m.m2d / m.n);
  out[4] = (m.m2a > 0.0 && m.m2b > 0.0) ? m.cab / sqrt(m.m2a * m.m2b) : __builtin_nan("");
}

hipError_t launch_prob_diff_stats(const float* a, const float* b, const uint8_t* mask, int64_t n, double* out,
                                  void* ws, hipStream_t s) {
  double* part = static_cast<double*>(ws);
  {
    TimedLaunch tl("k_prob_diff_stats", s);
    hipLaunchKernelGGL(k_prob_diff_stats_partial, dim3(kStatsBlocks), dim3(256), 0, s, a, b, mask, n, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_prob_diff_stats_final, dim3(1), dim3(64), 0, s, static_cast<const double*>(part),
                     kStatsBlocks, out);
  return hipGetLastError();
}

}  // namespace lp
