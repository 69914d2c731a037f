// bf16 MFMA GEMM mainloop for gfx950, both operands K-contiguous ("NT"):
//   D[m][n] = sum_k A[m][k] * B[n][k]
// A rows come from a row-major matrix (row m at a + m * lda); B rows are
// either contiguous or gathered through an index list (the scored rows of the
// hidden states).  Accumulators are fp32 and stay in registers; the caller's
// epilogue consumes them.
//
// Tiling: a workgroup of NT = 64 * WGM * WGN threads computes a BM x BN tile;
// wave (wm, wn) owns a (BM / WGM) x (BN / WGN) sub-tile made of 32x32
// v_mfma_f32_32x32x16_bf16 tiles.  K advances BK at a time through two LDS
// buffers: while the waves multiply out of one buffer, the next K-slice is
// already in flight from global memory into registers, then stored to the
// other buffer.  Rows of the LDS tiles are padded by 16 bytes so that the
// 32 lanes reading one operand column hit distinct banks.
//
// Accumulator layout of one 32x32 tile (lane l, register i, 0..15):
//   row m = 8 * (i / 4) + 4 * (l / 32) + (i % 4),   column n = l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr int NT = 64 * WGM * WGN;
  static constexpr int WTM = BM / WGM;  // wave tile rows
  static constexpr int WTN = BN / WGN;  // wave tile cols
  static constexpr int MI = WTM / 32;
  static constexpr int NI = WTN / 32;
  static constexpr int LDK = BK + 8;    // padded LDS row (bf16 elements)
  static constexpr int KC = BK / 8;     // 16-byte chunks per row
  static constexpr int A_CHUNKS = BM * KC / NT;
  static constexpr int B_CHUNKS = BN * KC / NT;
  static constexpr int LDS_ELEMS = 2 * (BM + BN) * LDK;
  static constexpr size_t LDS_BYTES = LDS_ELEMS * 2;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert((BM * KC) % NT == 0 && (BN * KC) % NT == 0, "tile not divisible among threads");
  static_assert(BK % 16 == 0, "BK must be a multiple of 16");
};

struct GemmOperands {
  const uint16_t* a;   // bf16 bits
  int64_t lda;
  int M;               // valid A rows (from m0 = 0)
  const uint16_t* b;
  int64_t ldb;
  const int* b_rows;   // gather list for B rows, or nullptr (identity)
  int N;               // valid B rows
  int K;               // multiple of 8
};

// Loads the global K-slice [k0, k0 + BK) of this block's A and B rows into
// registers (zero outside the valid range).
template <class C>
struct GemmStage {
  uint4 a[C::A_CHUNKS];
  uint4 b[C::B_CHUNKS];
};

template <class C>
__device__ __forceinline__ void gemm_load(GemmStage<C>& st, const GemmOperands& op, int m0, int n0, int k0,
                                          const int64_t* a_off, const int64_t* b_off) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int id = tid + i * C::NT;
    const int kc = id % C::KC;
    const int k = k0 + kc * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (a_off[i] >= 0 && k < op.K) v = *reinterpret_cast<const uint4*>(op.a + a_off[i] + k);
    st.a[i] = v;
  }
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) {
    const int id = tid + i * C::NT;
    const int kc = id % C::KC;
    const int k = k0 + kc * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (b_off[i] >= 0 && k < op.K) v = *reinterpret_cast<const uint4*>(op.b + b_off[i] + k);
    st.b[i] = v;
  }
}

template <class C>
__device__ __forceinline__ void gemm_store_lds(const GemmStage<C>& st, uint16_t* As, uint16_t* Bs) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int id = tid + i * C::NT;
    const int row = id / C::KC, kc = id % C::KC;
    *reinterpret_cast<uint4*>(As + row * C::LDK + kc * 8) = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) {
    const int id = tid + i * C::NT;
    const int row = id / C::KC, kc = id % C::KC;
    *reinterpret_cast<uint4*>(Bs + row * C::LDK + kc * 8) = st.b[i];
  }
}

template <class C>
__device__ __forceinline__ void gemm_compute(const uint16_t* As, const uint16_t* Bs, f32x16_t (&acc)[C::MI][C::NI],
                                             int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31;
  const int kh = (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < C::BK; kk += 16) {
    bf16x8_t af[C::MI], bfr[C::NI];
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
      af[mi] = *reinterpret_cast<const bf16x8_t*>(As + (wm * C::WTM + mi * 32 + r32) * C::LDK + kk + kh);
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
      bfr[ni] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * C::WTN + ni * 32 + r32) * C::LDK + kk + kh);
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < C::NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
  }
}

// Full K loop for the tile at (m0, n0).  `lds` must hold C::LDS_ELEMS bf16.
template <class C>
__device__ __forceinline__ void gemm_tile(const GemmOperands& op, int m0, int n0, uint16_t* lds,
                                          f32x16_t (&acc)[C::MI][C::NI]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int wm = wave % C::WGM, wn = wave / C::WGM;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  // per-thread row offsets (elements) of the chunks it loads; -1 = outside
  int64_t a_off[C::A_CHUNKS], b_off[C::B_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int row = (tid + i * C::NT) / C::KC;
    const int m = m0 + row;
    a_off[i] = (m < op.M) ? static_cast<int64_t>(m) * op.lda : -1;
  }
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) {
    const int row = (tid + i * C::NT) / C::KC;
    const int n = n0 + row;
    if (n < op.N) {
      const int64_t src = op.b_rows ? static_cast<int64_t>(op.b_rows[n]) : static_cast<int64_t>(n);
      b_off[i] = src * op.ldb;
    } else {
      b_off[i] = -1;
    }
  }

  uint16_t* As0 = lds;
  uint16_t* Bs0 = lds + C::BM * C::LDK;
  uint16_t* As1 = lds + (C::BM + C::BN) * C::LDK;
  uint16_t* Bs1 = As1 + C::BM * C::LDK;

  const int nk = (op.K + C::BK - 1) / C::BK;
  GemmStage<C> stg;
  gemm_load<C>(stg, op, m0, n0, 0, a_off, b_off);
  gemm_store_lds<C>(stg, As0, Bs0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gemm_load<C>(stg, op, m0, n0, (kt + 1) * C::BK, a_off, b_off);
    if (kt & 1)
      gemm_compute<C>(As1, Bs1, acc, wm, wn);
    else
      gemm_compute<C>(As0, Bs0, acc, wm, wn);
    if (more) {
      if (kt & 1)
        gemm_store_lds<C>(stg, As0, Bs0);
      else
        gemm_store_lds<C>(stg, As1, Bs1);
    }
    __syncthreads();
  }
}

// blockIdx -> logical tile id such that each XCD (hardware assigns workgroup
// b to XCD b % 8) works through one contiguous range of logical ids.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int q = n / 8, rem = n % 8;
  const int x = b % 8, j = b / 8;
  return (x < rem) ? x * (q + 1) + j : rem * (q + 1) + (x - rem) * q + j;
}

}  // namespace lp
