// bf16 MFMA GEMM mainloops for gfx950:
//   D[m][n] = sum_k A[m][k] * B[n][k]
// The generic loop (gemm_tile) takes K-contiguous ("NT") operands: A rows
// from a row-major matrix (row m at a + m * lda), B rows contiguous or
// gathered through an index list (the scored rows of the hidden states).  The
// fast loop further down (gemm_tile_dtl*) also takes K-major operands.
// Accumulators are fp32 and stay in registers; the caller's epilogue
// consumes them.
//
// Generic tiling: a workgroup of NT = 64 * WGM * WGN threads computes a BM x BN tile;
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

#include <type_traits>

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


// ---------------------------------------------------------------------------
// Fast mainloop for K % BK == 0: global -> LDS with buffer_load_dwordx4 ...
// lds (no register staging), XOR-swizzled LDS rows, NS LDS stages, fragment
// prefetch one K-substep ahead.
//
// Each operand is either K-contiguous ("NT", element (m, k) at m * ld + k)
// or K-major (element (m, k) at k * ld + m: the m index is contiguous).
//
// K-contiguous operand: LDS row = one m, BK bf16 = KC chunks of 16 bytes; the
// chunk holding logical 16-byte column kc of row r sits at position
// kc ^ swz(r), so the 32 lanes reading one fragment column (rows r..r+31,
// same kc) spread over all banks:
//   BK = 64 (128-byte rows): swz(r) = (r & 7) ^ ((r >> 3) & 1);
//   BK = 32 (64-byte rows, two rows per 128-byte bank line): swz(r) = (r >> 1) & 3.
// K-major operand: LDS row = one k, ROWS (= BM or BN) bf16 = ROWS / 8 chunks;
// chunk mc of row k sits at mc ^ (4 (k & 3)).  Its MFMA fragments come from
// gfx950's transposing LDS read (ds_read_b64_tr_b16): within each 16-lane
// group, lane (r, c) = ((lane & 15) >> 2, lane & 3) names 4 consecutive
// elements of row r, and after the read lane j holds element j of each of
// the 4 rows; two reads give a lane its 8 consecutive k of one m, the layout
// the MFMA takes.  With the swizzle the 16 (row, chunk) pairs a half-wave
// touches fall in distinct banks.
// Each wave-wide load instruction fills 64 consecutive chunk slots (1 KB), so
// every lane loads the global chunk that belongs in its slot.
// Rows (K-contiguous) or chunks (K-major) past the valid range are clamped to
// the last valid one (their results are discarded by the caller); K-major
// rows past `kvalid` are clamped likewise.  K must be a multiple of BK.
// ---------------------------------------------------------------------------

#ifndef LP_FRAG_PER_SLOT
#define LP_FRAG_PER_SLOT 2
#endif

typedef __attribute__((address_space(3))) void lds_void_t;

template <int BM_, int BN_, int WGM_, int WGN_, int BK_ = 64, int NS_ = 2, bool AKM_ = false, bool BKM_ = false>
struct DtlCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr int NS = NS_;                      // LDS stages
  static constexpr bool AKM = AKM_, BKM = BKM_;       // K-major operands
  static constexpr int NT = 64 * WGM * WGN;
  static constexpr int NW = WGM * WGN;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int MI = WTM / 32, NI = WTN / 32;
  static constexpr int KC = BK / 8;                   // 16-byte chunks per row
  // Waves that issue the global loads.  With two waves per SIMD, letting only
  // one of them load keeps the other free to feed the matrix unit while the
  // loads queue.
#ifdef LP_LOADER_WAVES
  static constexpr int LW = LP_LOADER_WAVES < NW ? LP_LOADER_WAVES : NW;
#else
  static constexpr int LW = NW >= 8 ? NW / 2 : NW;
#endif
  static constexpr int A_INST = BM * KC / 64 / LW;    // load instructions per loading wave per stage (A)
  static constexpr int B_INST = BN * KC / 64 / LW;
  static constexpr int STAGE_ELEMS = (BM + BN) * BK;
  static constexpr int LDS_ELEMS = NS * STAGE_ELEMS;
  // B fragments reloaded in place after their last use (one register set
  // instead of two) when the accumulators plus two fragment sets would not
  // fit two waves per SIMD.
#ifdef LP_FRAG_B_INPLACE
  static constexpr bool B_INPLACE = LP_FRAG_B_INPLACE != 0;
#else
  static constexpr bool B_INPLACE = MI * NI * 16 + 8 * (MI + NI) > 224;
#endif
  static constexpr int FB_SETS = B_INPLACE ? 1 : 2;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert((BM * KC) % (64 * LW) == 0 && (BN * KC) % (64 * LW) == 0, "tile not divisible among waves");
  static_assert(BK == 64 || BK == 32, "LDS swizzle defined for 64- and 128-byte rows");
  static_assert(NS >= 2 && (NS & (NS - 1)) == 0, "stage count must be a power of two >= 2");
  static_assert(!AKM || (BM % 128 == 0 && BK % 16 == 0), "K-major A: rows of at least 16 chunks");
  static_assert(!BKM || (BN % 128 == 0 && BK % 16 == 0), "K-major B: rows of at least 16 chunks");
};

__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int KC>
__device__ __forceinline__ int lds_swz_k(int r) {
  if constexpr (KC == 8)
    return lds_swz(r);
  else
    return (r >> 1) & 3;
}

// K-major rows: chunk position of logical chunk mc in LDS row k is mc ^ lds_swz_km(k).
__device__ __forceinline__ int lds_swz_km(int k) { return 4 * (k & 3); }

// Row sources of one operand for this thread: a buffer resource on the
// operand base and the byte offset of the global chunk each of its load
// instructions moves; the stage's K offset (kstart x kstride bytes) goes in
// the scalar offset, so a load needs no vector address arithmetic.
// The buffer-resource type exists only in the device pass; the host pass
// parses device code without generating it.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t dtl_rsrc_t;
#else
struct dtl_rsrc_t {
  unsigned w[4];
};
#endif

// LIN (dense K-contiguous rows): instruction j's rows are instruction 0's plus
// j x LW x (64 / KC) rows, all with the same 16-byte chunk, so one offset, a
// uniform step and a per-lane clamp describe them all (fewer live registers).
template <int NINST, bool LIN = false>
struct DtlRows {
  static constexpr int N = NINST;
  dtl_rsrc_t rsrc;
  uint32_t off[LIN ? 1 : NINST];  // byte offsets from the operand base (the caller checks they fit in 32 bits)
  uint32_t jstride;               // LIN: bytes from one instruction's rows to the next's (uniform)
  uint32_t offmax;                // LIN: offset of this lane's chunk in the last valid row
  uint32_t kstride;               // bytes per unit of K: 2 (K-contiguous) or ld * 2 (K-major)
  int kvalid;                     // K-major: rows of K that exist (the rest are clamped to the last)
  __device__ __forceinline__ uint32_t at(int j) const {
    if constexpr (LIN) {
      const uint32_t o = off[0] + static_cast<uint32_t>(j) * jstride;
      return o < offmax ? o : offmax;
    } else {
      return off[j];
    }
  }
};

// Raw buffer over [base, base + 4 GiB): offsets are kept in range by the row
// clamping, the descriptor only removes the 64-bit address arithmetic.
// Word 3 selects 32-bit data format, as untyped gfx9 buffer loads expect.
__device__ __forceinline__ dtl_rsrc_t dtl_rsrc(const void* base) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(0xffffffffu),
                                           0x00020000);
#else
  (void)base;
  return dtl_rsrc_t{};
#endif
}

// 16-byte chunk at rsrc + voff + soff into this lane's slot of the 1 KB LDS
// block at dst (direct to LDS, no staging registers).
__device__ __forceinline__ void dtl_load16(const dtl_rsrc_t& rsrc, uint16_t* dst, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst), 16, voff, soff, 0, 0);
#else
  (void)rsrc, (void)dst, (void)voff, (void)soff;
#endif
}

// K-contiguous operand: rows m0 + r of a row-major matrix (clamped to M - 1).
// Instruction j moves rows r0 + j x LW x (64 / KC) with the lane's chunk kc;
// the swizzle of a row depends only on row bits that j does not change (LW
// even for 8 chunks per row, any LW for 4), so kc is the same for every j and
// the clamp to row M - 1 is a clamp of the offset.
template <class C, int NINST>
__device__ __forceinline__ void dtl_rows_dense(DtlRows<NINST, true>& rw, int64_t ld, int M) {
  static_assert(C::KC == 4 || C::LW % 2 == 0, "chunk swizzle must not depend on the instruction index");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = wave * 64 + lane;
  const int r = slot / C::KC, pc = slot % C::KC;
  const int kc = pc ^ lds_swz_k<C::KC>(r);
  const int rr = r < M ? r : M - 1;
  rw.off[0] = static_cast<uint32_t>((static_cast<int64_t>(rr) * ld + kc * 8) * 2);
  rw.offmax = static_cast<uint32_t>((static_cast<int64_t>(M - 1) * ld + kc * 8) * 2);
  rw.jstride = static_cast<uint32_t>(static_cast<int64_t>(C::LW * (64 / C::KC)) * ld * 2);
  rw.kstride = 2;
  rw.kvalid = 0x7fffffff;
}

// K-contiguous operand, gathered rows rows[r], or rows r when rows is null (clamped to N - 1).
template <class C, int NINST>
__device__ __forceinline__ void dtl_rows_gather(DtlRows<NINST>& rw, int64_t ld, const int* rows, int N) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < NINST; ++j) {
    const int slot = (j * C::LW + wave) * 64 + lane;
    const int r = slot / C::KC, pc = slot % C::KC;
    const int kc = pc ^ lds_swz_k<C::KC>(r);
    const int rr = r < N ? r : N - 1;
    const int64_t src = rows ? static_cast<int64_t>(rows[rr]) : static_cast<int64_t>(rr);
    rw.off[j] = static_cast<uint32_t>((src * ld + kc * 8) * 2);
  }
  rw.kstride = 2;
  rw.kvalid = 0x7fffffff;
}

// K-major operand of ROWS (= BM or BN) m-columns per LDS row: element (m, k)
// at base + k * ld + m; columns from `mvalid` on are clamped to the last valid
// 8-column chunk, K rows from `kvalid` on to row kvalid - 1 (at issue time).
template <class C, int NINST, int ROWS>
__device__ __forceinline__ void dtl_rows_km(DtlRows<NINST>& rw, int64_t ld, int mvalid, int kvalid) {
  constexpr int CPR = ROWS / 8;  // chunks per LDS row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cmax = (mvalid - 1) >> 3;
#pragma unroll
  for (int j = 0; j < NINST; ++j) {
    const int slot = (j * C::LW + wave) * 64 + lane;
    const int k = slot / CPR, pc = slot % CPR;
    int mc = pc ^ lds_swz_km(k);
    mc = mc < cmax ? mc : cmax;
    rw.off[j] = static_cast<uint32_t>((static_cast<int64_t>(k) * ld + mc * 8) * 2);
  }
  rw.kstride = static_cast<uint32_t>(ld * 2);
  rw.kvalid = kvalid;
}

// 8 bf16 of one K-major fragment: rows kk + 8 (g >> 1) + [0, 8) of column
// mb + 16 (g & 1) + (lane & 15), g = lane >> 4, from an LDS stage region of
// ROWS columns per row -- the MFMA operand layout (lane l: m = l % 32,
// k = 8 (l / 32) + [0, 8)).
//
// The two reads are issued as inline assembly: through the compiler builtin,
// the compiler cannot tell them from the in-flight direct-to-LDS loads of
// other stages and waits for all global loads before each one.  The
// compiler therefore does not track these reads either; the K loop waits for
// them itself (dtl_wait_frags before the MFMAs that use them, and before each
// stage barrier, so no read of a stage is in flight once it is reloaded).
template <int ROWS>
__device__ __forceinline__ bf16x8_t dtl_frag_km(const uint16_t* region, int kk, int mb) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
  const int m = mb + 16 * (g & 1) + 4 * c;
  const int k0 = kk + 8 * (g >> 1) + r;
  const int pos = (((m >> 3) ^ lds_swz_km(r)) << 3) + (m & 7);  // k0 & 3 == r
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)(region + k0 * ROWS + pos)));
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  u32x2_t lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(a));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(a), "i"(4 * ROWS * 2));
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

// Waits until every LDS read this wave issued has returned; the fragment
// registers are tied to the wait so that no MFMA reading them is scheduled
// before it.  Needed only when a fragment comes from dtl_frag_km.
template <class C>
__device__ __forceinline__ void dtl_wait_frags(bf16x8_t (&fa)[C::MI], bf16x8_t (&fb)[C::NI]) {
  if constexpr (C::AKM || C::BKM) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < C::MI; ++i) asm volatile("" : "+v"(fa[i]));
#pragma unroll
    for (int i = 0; i < C::NI; ++i) asm volatile("" : "+v"(fb[i]));
  }
}

// One fragment: piece q < MI reads A fragment q, else B fragment q - MI.
template <class C>
__device__ __forceinline__ void dtl_frag_piece(const uint16_t* stage, int kk, int wm, int wn, int q,
                                               bf16x8_t (&af)[C::MI], bf16x8_t (&bfr)[C::NI]) {
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31;
  const int pc = ((kk >> 3) + (lane >> 5)) ^ lds_swz_k<C::KC>(r32);
  if (q < C::MI) {
    if constexpr (C::AKM)
      af[q] = dtl_frag_km<C::BM>(stage, kk, wm * C::WTM + q * 32);
    else
      af[q] = *reinterpret_cast<const bf16x8_t*>(stage + (wm * C::WTM + q * 32 + r32) * C::BK + pc * 8);
  } else {
    const int ni = q - C::MI;
    if constexpr (C::BKM)
      bfr[ni] = dtl_frag_km<C::BN>(stage + C::BM * C::BK, kk, wn * C::WTN + ni * 32);
    else
      bfr[ni] = *reinterpret_cast<const bf16x8_t*>(stage + (C::BM + wn * C::WTN + ni * 32 + r32) * C::BK + pc * 8);
  }
}

// Per-lane offset of load instruction j of a K-major operand for the stage
// starting at K index kstart: rows past kvalid - 1 are moved back to it
// (only in a stage that reaches past kvalid; the test is uniform).
template <class C, int NINST, int ROWS>
__device__ __forceinline__ uint32_t dtl_km_off(const DtlRows<NINST, false>& rw, int j, int kstart, int wave) {
  uint32_t voff = rw.off[j];
  if (kstart + C::BK > rw.kvalid) {
    const int lane = threadIdx.x & 63;
    const int k = ((j * C::LW + wave) * 64 + lane) / (ROWS / 8);
    const int over = kstart + k - (rw.kvalid - 1);
    if (over > 0) voff -= static_cast<uint32_t>(over) * rw.kstride;
  }
  return voff;
}

// Issue global load instruction j (A for j < A_INST, else B) of the stage
// starting at K index kstart; the per-lane part is a 32-bit offset, the
// stage's K offset a scalar one.  Only the first LW waves load (see DtlCfg::LW).
template <class C, class RA, class RB>
__device__ __forceinline__ void dtl_issue_one(int j, int kstart, const RA& ra, const RB& rb, uint16_t* stage,
                                              int wave) {
  constexpr int NA = RA::N;
  // `wave` is the uniform (scalar) wave index, so the LDS destination (M0) is scalar arithmetic
  if (j < NA) {
    uint16_t* dst = stage + (j * C::LW + wave) * 64 * 8;
    uint32_t voff;
    if constexpr (C::AKM)
      voff = dtl_km_off<C, NA, C::BM>(ra, j, kstart, wave);
    else
      voff = ra.at(j);
    dtl_load16(ra.rsrc, dst, voff, static_cast<uint32_t>(kstart) * ra.kstride);
  } else {
    const int jb = j - NA;
    uint16_t* dst = stage + C::BM * C::BK + (jb * C::LW + wave) * 64 * 8;
    uint32_t voff;
    if constexpr (C::BKM)
      voff = dtl_km_off<C, RB::N, C::BN>(rb, jb, kstart, wave);
    else
      voff = rb.at(jb);
    dtl_load16(rb.rsrc, dst, voff, static_cast<uint32_t>(kstart) * rb.kstride);
  }
}
// Wait until at most `pending` stages' worth of this wave's global loads are
// still in flight (pending is uniform and at most 3).
template <class C>
__device__ __forceinline__ void dtl_wait_vm(int pending) {
  constexpr int NL = C::A_INST + C::B_INST;
  static_assert(3 * NL <= 63, "vmcnt field is 6 bits");
  if (pending <= 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (pending == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");
  else if (pending == 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NL) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * NL) : "memory");
}

// One K-step on stage X (the next stage is Y).  Instruction order, fixed with
// scheduling barriers so that an MFMA never waits on a fragment read issued
// just before it:
//   substeps 0 .. S-2: MFMAs on X; between them, the fragment reads of the next
//                      substep (from X).
//   end of S-2:        wait for this wave's loads of the next stage (`pending`
//                      later stages may stay in flight), barrier (next stage
//                      complete in Y; every wave is done reading X).
//   substep S-1:       MFMAs on X (fragments already in registers); between them,
//                      the first fragments of the next stage (from Y) and the
//                      global loads of the stage NS steps ahead (into X),
//                      which starts at K index k2.
template <class C, bool NEXT, bool NEXT2, class RA, class RB>
__device__ __forceinline__ void dtl_kstep(uint16_t* X, uint16_t* Y, int k2, const RA& ra,
                                          const RB& rb, int wm, int wn,
                                          bf16x8_t (&fa)[2][C::MI], bf16x8_t (&fb)[2][C::NI],
                                          f32x16_t (&acc)[C::MI][C::NI], int pending, int wave) {
  constexpr int S = C::BK / 16;
  constexpr int NQ = C::MI * C::NI;
  constexpr int NF = C::MI + C::NI;
  constexpr int NL = C::A_INST + C::B_INST;
  static_assert(S % 2 == 0, "substep 0 of every stage must use fragment buffer 0");
  constexpr int PER = LP_FRAG_PER_SLOT;  // fragment reads between two MFMAs
  static_assert(NF <= PER * NQ, "not enough MFMA slots to interleave fragment reads");
  const bool loader = C::LW == C::NW || wave < C::LW;  // scalar test; compile-time true when every wave loads
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int cur = s & 1;
    dtl_wait_frags<C>(fa[cur], fb[cur]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      // fragment reads of the next substep, PER per MFMA slot from the start
      // of the substep, so they have most of it to land
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int f = PER * q + u;
        if (f < NF) {
          if (s + 1 < S)
            dtl_frag_piece<C>(X, (s + 1) * 16, wm, wn, f, fa[cur ^ 1], fb[cur ^ 1]);
          else if (NEXT)
            dtl_frag_piece<C>(Y, 0, wm, wn, f, fa[cur ^ 1], fb[cur ^ 1]);
        }
      }
      if (s + 1 == S && NEXT2 && loader) {
        // the loads of the stage after next, spread over this substep
#pragma unroll
        for (int u = 0; u < (NL + NQ - 1) / NQ; ++u) {
          const int j = q * ((NL + NQ - 1) / NQ) + u;
          if (j < NL) dtl_issue_one<C>(j, k2, ra, rb, X, wave);
        }
      }
      const int mi = q / C::NI, ni = q % C::NI;
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][mi], fb[cur][ni], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (NEXT && s == S - 2) {
      dtl_wait_frags<C>(fa[cur ^ 1], fb[cur ^ 1]);
      dtl_wait_vm<C>(pending);
      __syncthreads();
    }
  }
}

// The same K-step with one B fragment set.  MFMAs run column by column
// (q = ni * MI + mi), so B fragment ni is free once column ni is done and its
// next-substep copy is read right then, into the same registers; the A
// fragments of the next substep go to the other A set in the first MI slots.
// The last column's B fragment is read after the substep's last MFMA, before
// the stage barrier, so no wave reads a stage that others may overwrite.
template <class C, bool NEXT, bool NEXT2, class RA, class RB>
__device__ __forceinline__ void dtl_kstep_bi(uint16_t* X, uint16_t* Y, int k2, const RA& ra,
                                             const RB& rb, int wm, int wn,
                                             bf16x8_t (&fa)[2][C::MI], bf16x8_t (&fb)[C::NI],
                                             f32x16_t (&acc)[C::MI][C::NI], int pending, int wave) {
  constexpr int S = C::BK / 16;
  constexpr int NQ = C::MI * C::NI;
  constexpr int NL = C::A_INST + C::B_INST;
  static_assert(S % 2 == 0, "substep 0 of every stage must use A fragment set 0");
  static_assert(!C::AKM && !C::BKM, "in-place B fragments: K-contiguous operands only");
  const bool loader = C::LW == C::NW || wave < C::LW;
  bf16x8_t dummy[C::MI];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int cur = s & 1;
    const bool rd = s + 1 < S || NEXT;  // fragments of a next substep exist
    uint16_t* src = s + 1 < S ? X : Y;
    const int kk = s + 1 < S ? (s + 1) * 16 : 0;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (rd && q < C::MI) dtl_frag_piece<C>(src, kk, wm, wn, q, fa[cur ^ 1], fb);
      if (rd && q >= C::MI && q % C::MI == 0)
        dtl_frag_piece<C>(src, kk, wm, wn, C::MI + q / C::MI - 1, dummy, fb);
      if (s + 1 == S && NEXT2 && loader) {
#pragma unroll
        for (int u = 0; u < (NL + NQ - 1) / NQ; ++u) {
          const int j = q * ((NL + NQ - 1) / NQ) + u;
          if (j < NL) dtl_issue_one<C>(j, k2, ra, rb, X, wave);
        }
      }
      const int ni = q / C::MI, mi = q % C::MI;
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][mi], fb[ni], acc[mi][ni], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (rd) dtl_frag_piece<C>(src, kk, wm, wn, C::MI + C::NI - 1, dummy, fb);
    if (NEXT && s == S - 2) {
      dtl_wait_vm<C>(pending);
      __syncthreads();
    }
  }
}

// The K loop of one block on prepared row sources (see gemm_tile_dtl and
// gemm_tile_dtl_dense below).  K is a multiple of BK and may be 0 (D = 0).
template <class C, class RA, class RB>
__device__ __forceinline__ void gemm_dtl_loop(const RA& ra, const RB& rb, int K,
                                              uint16_t* lds, f32x16_t (&acc)[C::MI][C::NI]) {
  constexpr int NF = C::MI + C::NI;
  constexpr int NL = C::A_INST + C::B_INST;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers
  const int wm = wave % C::WGM, wn = wave / C::WGM;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;
  const int nk = K / C::BK;
  if (nk <= 0) return;  // empty K: D = 0
  // prologue: the first min(NS, nk) stages in flight, wait for stage 0, read its first fragments
  const int npro = nk < C::NS ? nk : C::NS;
  if (C::LW == C::NW || wave < C::LW) {
#pragma unroll
    for (int st = 0; st < C::NS; ++st) {
      if (st < npro) {
#pragma unroll
        for (int j = 0; j < NL; ++j)
          dtl_issue_one<C>(j, st * C::BK, ra, rb, lds + st * C::STAGE_ELEMS, wave);
      }
    }
    dtl_wait_vm<C>(npro - 1);
  }
  __syncthreads();
  bf16x8_t fa[2][C::MI], fb[C::FB_SETS][C::NI];
#pragma unroll
  for (int q = 0; q < NF; ++q) dtl_frag_piece<C>(lds, 0, wm, wn, q, fa[0], fb[0]);

  auto stage = [&](int k) { return lds + (k & (C::NS - 1)) * C::STAGE_ELEMS; };
  auto kstep = [&](auto next, auto next2, int kt, int k2, int pending) {
    if constexpr (C::B_INPLACE)
      dtl_kstep_bi<C, decltype(next)::value, decltype(next2)::value>(stage(kt), stage(kt + 1), k2, ra, rb, wm, wn,
                                                                     fa, fb[0], acc, pending, wave);
    else
      dtl_kstep<C, decltype(next)::value, decltype(next2)::value>(stage(kt), stage(kt + 1), k2, ra, rb, wm, wn, fa,
                                                                  fb, acc, pending, wave);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int kt = 0;
  // steady state: stage kt + NS is loaded into stage kt's buffer; NS - 2 later stages stay in flight
  for (; kt + C::NS < nk; ++kt) kstep(T_{}, T_{}, kt, (kt + C::NS) * C::BK, C::NS - 2);
  // drain: no more loads; stages kt + 2 .. nk - 1 are still in flight
  for (; kt + 1 < nk; ++kt) kstep(T_{}, F_{}, kt, 0, nk - kt - 2);
  kstep(F_{}, F_{}, kt, 0, 0);
  __syncthreads();
}

// D[m][n] = sum_k A[m][k] * B[rows[n]][k] over K (multiple of 64, may be 0),
// both operands K-contiguous.  a: bf16 rows of the block (row 0 = the block's
// first row, column 0 = the first K column used), M valid rows; b: bf16 base
// of the gathered matrix, b_rows the gather list (null: rows 0..N-1 of b), N
// valid rows.  Byte offsets of every row read from a and b must fit in 32 bits.
template <class C>
__device__ __forceinline__ void gemm_tile_dtl(const uint16_t* a, int64_t lda, int M, const uint16_t* b,
                                              int64_t ldb, const int* b_rows, int N, int K, uint16_t* lds,
                                              f32x16_t (&acc)[C::MI][C::NI]) {
  static_assert(!C::AKM && !C::BKM, "K-contiguous operands");
  DtlRows<C::A_INST, true> ra;
  DtlRows<C::B_INST> rb;
  dtl_rows_dense<C, C::A_INST>(ra, lda, M);
  dtl_rows_gather<C, C::B_INST>(rb, ldb, b_rows, N);
  ra.rsrc = dtl_rsrc(a);
  rb.rsrc = dtl_rsrc(b);
  gemm_dtl_loop<C>(ra, rb, K, lds, acc);
}

// D[m][n] = sum_k A(m, k) * B(n, k) over K (multiple of 64, may be 0) on
// dense operands, each K-contiguous or K-major as C::AKM / C::BKM say:
//   K-contiguous: element (m, k) at a + m * lda + k, M valid rows;
//   K-major:      element (m, k) at a + k * lda + m, M valid columns, and
//                 rows k >= kvalid_a clamped to kvalid_a - 1 (zero
//                 multipliers on the other side must make them irrelevant).
// a and b point at the block's element (0, 0).  Every per-lane byte offset
// (one BM- or BN-row block of a K-contiguous operand, BK rows of a K-major
// one) and K x the K-major pitch in bytes must fit in 32 bits.
template <class C>
__device__ __forceinline__ void gemm_tile_dtl_dense(const uint16_t* a, int64_t lda, int M, int kvalid_a,
                                                    const uint16_t* b, int64_t ldb, int N, int kvalid_b, int K,
                                                    uint16_t* lds, f32x16_t (&acc)[C::MI][C::NI]) {
  DtlRows<C::A_INST, !C::AKM> ra;
  DtlRows<C::B_INST, !C::BKM> rb;
  if constexpr (C::AKM)
    dtl_rows_km<C, C::A_INST, C::BM>(ra, lda, M, kvalid_a);
  else
    dtl_rows_dense<C, C::A_INST>(ra, lda, M);
  if constexpr (C::BKM)
    dtl_rows_km<C, C::B_INST, C::BN>(rb, ldb, N, kvalid_b);
  else
    dtl_rows_dense<C, C::B_INST>(rb, ldb, N);
  ra.rsrc = dtl_rsrc(a);
  rb.rsrc = dtl_rsrc(b);
  gemm_dtl_loop<C>(ra, rb, K, lds, acc);
}

}  // namespace lp
