// Fused LM head on gfx950: forward log-prob / entropy and the
// recompute-based backward, without a [rows x vocab] logits buffer.
//
// miles PR #4645 ("How it works"): the scored rows are selected before the
// output layer (prompt rows are never multiplied by the weight), processed a
// tile of rows at a time, and the backward replays each tile.  Here:
//
//   k_compact       mask -> ascending scored-row list idx[] + count (device
//                   side, so the host never waits); zero-fills the per-row
//                   outputs of unscored rows.
//   k_fwd_tile      per tile: MFMA GEMM logits^T = W . H_tile^T with vocab as
//                   the MFMA row dimension, so each lane's accumulators hold
//                   one token's logits for 16 vocab rows per 32x32 tile; the
//                   epilogue folds them into that token's (mc, s, a) state in
//                   registers, merges across lanes / waves and writes one
//                   partial state per (row, vocab block), plus the target
//                   logit from the block that owns the target column.
//   k_fwd_merge     merges a row's partial states in a fixed order and writes
//                   log-prob, entropy and log-sum-exp.
//   backward        k_bwd_dz recomputes the tile's logits with the same GEMM
//                   and writes dL/dlogits (bf16) as dZ [row][vocab];
//                   dHidden (= dZ . W, K = vocab, split over K) reads the
//                   weight as stored (a K-major operand) and dW (+= dZ^T .
//                   H, K = the rows of two consecutive tiles) reads dZ and a
//                   dense copy of the tiles' hidden rows as K-major operands,
//                   through the LDS transposing reads.  The generic tiles
//                   (h % 64 != 0) write dZ in both orders and multiply
//                   against transposed copies of W and of the tile's rows.
//   KL              both models' heads: see the KL section below.
#include "lp_device.hpp"
#include "lp_gemm.hpp"
#include "lp_internal.hpp"

namespace lp {

namespace {

constexpr float kLog2eF = 1.44269504088896340736f;

// Block tiles (BM, BN, BK, waves along M, waves along N); build-time knobs.
#ifndef LP_FWD_TILE
#define LP_FWD_TILE 128, 128, 64, 2, 2
#endif
#ifndef LP_BWD_TILE
#define LP_BWD_TILE 128, 128, 64, 2, 2
#endif
using FwdCfg = GemmCfg<LP_FWD_TILE>;
#ifndef LP_FWD_DTL_TILE
#define LP_FWD_DTL_TILE 256, 320, 4, 2
#endif
// Minimum waves per SIMD the forward tile is compiled for (register budget).
#ifndef LP_FWD_MIN_WAVES
#define LP_FWD_MIN_WAVES 1
#endif
using FwdDtlCfg = DtlCfg<LP_FWD_DTL_TILE>;
// Row tiles per launch of the fast forward: blocks of consecutive tiles run
// back to back instead of each launch ending on a partly filled last wave of
// blocks (measured 2.5 % of the forward with one tile per launch).
#ifndef LP_FWD_TILES_PER_LAUNCH
#define LP_FWD_TILES_PER_LAUNCH 8
#endif
constexpr int kFwdTilesPerLaunch = LP_FWD_TILES_PER_LAUNCH;
// Backward GEMMs on the fast path (dL/dlogits recompute, dHidden, dW).
#ifndef LP_BWD_DTL_TILE
#define LP_BWD_DTL_TILE 256, 256, 4, 2
#endif
using BwdDtlCfg = DtlCfg<LP_BWD_DTL_TILE>;
// The backward's dense gradient GEMMs (N is the hidden width), straight on
// the dZ buffer [rows][vocab] and the weight / the tile's hidden rows as
// stored: dHidden = dZ . W takes W as a K-major operand (its rows are the K
// index), dW = dZ^T . H_tile takes both operands K-major (K = the tile's rows).
#ifndef LP_DENSE_DTL_TILE
#define LP_DENSE_DTL_TILE 256, 256, 4, 2
#endif
using DenseDhCfg = DtlCfg<LP_DENSE_DTL_TILE, 64, 2, false, true>;
using DenseDwCfg = DtlCfg<LP_DENSE_DTL_TILE, 64, 2, true, true>;
using DenseDtlCfg = DenseDhCfg;  // block shape shared by both
// KL through both heads on the fast path: two passes per chunk of at most
// kKLChunk scored rows on this tile.  The teacher pass stores its fp32 logits
// for the chunk; the student pass's epilogue reads them back.  Measured on
// the 16384 x 7168 x 129280 distillation shape: 4096-row chunks beat 2048 and
// 1024 (each chunk re-reads both weights) and the one-kernel form with both
// accumulator sets, which caps the wave tile at 128 x 64.
#ifndef LP_KL_TILE
#define LP_KL_TILE 256, 256, 4, 2
#endif
using KLCfg = DtlCfg<LP_KL_TILE>;
#ifndef LP_KL_CHUNK_ROWS
#define LP_KL_CHUNK_ROWS 4096
#endif
constexpr int kKLChunk = LP_KL_CHUNK_ROWS;
static_assert(kKLChunk % KLCfg::BN == 0 && kKLChunk % 64 == 0, "chunk must hold whole row blocks");

// K splits of the dHidden GEMM (its output is only tile_rows x h, too few
// blocks to fill the chip without splitting K = V).
constexpr int kSplitK = 4;
using BwdCfg = GemmCfg<LP_BWD_TILE>;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_pk_t __attribute__((ext_vector_type(2)));

// Four fp32 values -> four bf16 (nearest even) packed in 8 bytes, with the
// hardware pair conversion.
__device__ __forceinline__ uint2 pack_bf16x4(const float (&d)[4]) {
  const bf16x2_pk_t lo = __builtin_convertvector(f32x2_t{d[0], d[1]}, bf16x2_pk_t);
  const bf16x2_pk_t hi = __builtin_convertvector(f32x2_t{d[2], d[3]}, bf16x2_pk_t);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Logical tile -> (vocab block, token block): groups of kGroupV vocab blocks
// sweep all token blocks, token-block-major inside a group, so consecutive
// workgroups on one XCD share both weight and hidden strips in its L2.
#ifndef LP_GROUP_V
#define LP_GROUP_V 4
#endif
constexpr int kGroupV = LP_GROUP_V;
template <int G = kGroupV>
__device__ __forceinline__ void tile_coords(int L, int n_vb, int n_nb, int& vb, int& nb) {
  const int full = n_vb / G;
  const int g = L / (G * n_nb);
  if (g < full) {
    const int w = L - g * G * n_nb;
    nb = w / G;
    vb = g * G + w % G;
  } else {
    const int w = L - full * G * n_nb;
    const int gsz = n_vb - full * G;
    nb = w / gsz;
    vb = full * G + w % gsz;
  }
}

// The direct-to-LDS loads address each operand through a buffer descriptor
// with a 32-bit per-lane byte offset (row r of pitch ld, plus the 16-byte
// chunk) and the stage's K offset added on top: `rows` rows of pitch `ld`
// plus a K span of `k` elements (bf16) must stay below 2^32 bytes.
bool u32_span(int64_t rows, int64_t ld, int64_t k) {
  return (static_cast<uint64_t>(rows) * static_cast<uint64_t>(ld) + static_cast<uint64_t>(k)) * 2u < (1ull << 32);
}

// Largest vocab (A) block of the direct-to-LDS GEMMs that read the weight.
constexpr int kDtlWeightRows = FwdDtlCfg::BM > BwdDtlCfg::BM ? (FwdDtlCfg::BM > KLCfg::BM ? FwdDtlCfg::BM : KLCfg::BM)
                                                              : (BwdDtlCfg::BM > KLCfg::BM ? BwdDtlCfg::BM : KLCfg::BM);

// Direct-to-LDS tiles for the logit GEMM of one head: K = h in steps of 64,
// the gathered hidden rows (any of the T rows) and one weight block of
// kDtlWeightRows rows within 32-bit offsets.
bool head_fast(int64_t T, int64_t h, int64_t ld_h, int64_t ld_w) {
  return h % FwdDtlCfg::BK == 0 && h % KLCfg::BK == 0 && u32_span(T, ld_h, h) && u32_span(kDtlWeightRows, ld_w, h);
}

// ... and for the backward's gradient GEMMs, per tile of tpad rows (tile_rows
// rounded up to 64) and vpad vocab columns (V rounded up to 64): dHidden reads
// 256-row blocks of dZ [rows][vpad] and the weight as a K-major operand (K
// index = vocab row, up to vpad rows of pitch ld_w); dW reads dZ and the
// tile's hidden rows [rows][h] as K-major operands over K = the rows of one
// tile, or of two (tiles_per_dw) when that also fits.
bool dense_fast(int64_t vpad, int64_t tpad, int64_t h, int64_t ld_w, int tiles_per_dw = 1) {
  constexpr int R = DenseDtlCfg::BM > DenseDtlCfg::BN ? DenseDtlCfg::BM : DenseDtlCfg::BN;
  const int64_t ksplit = static_cast<int64_t>(align_up(static_cast<size_t>((vpad + kSplitK - 1) / kSplitK), 64));
  const int64_t kt = tiles_per_dw * tpad;
  return u32_span(R, vpad, vpad) && u32_span(ksplit, ld_w, R) && u32_span(kt, vpad, R) && u32_span(kt, h, R);
}

bool lmhead_fast_path(const LMHeadShape& sh) { return head_fast(sh.T, sh.h, sh.ld_h, sh.ld_w); }

int64_t bwd_tpad(int64_t T, int64_t tile_rows) {
  const int64_t tr = tile_rows < T ? tile_rows : T;
  return static_cast<int64_t>(align_up(static_cast<size_t>(tr > 0 ? tr : 1), 64));
}

}  // namespace

bool lmhead_fast_tiles(int64_t T, int64_t h, int64_t V, int64_t ld_h, int64_t ld_w, int64_t tile_rows,
                       int backward) {
  if (!head_fast(T, h, ld_h, ld_w)) return false;
  if (!backward) return true;
  return dense_fast(static_cast<int64_t>(align_up(static_cast<size_t>(V), 64)), bwd_tpad(T, tile_rows), h, ld_w);
}

// The backward's buffers from the workspace base + dz_off.  Generic tiles: dZ,
// dZ^T, W^T, H_tile^T, dHidden partials.  Direct-to-LDS tiles: the dZ of two
// consecutive tiles (the dW GEMM runs once per pair, with K = both tiles'
// rows) and the two tiles' hidden rows, dHidden partials.  The scratch is the
// larger of the two, so either path runs in a workspace sized for the call.
struct BwdBuffers {
  uint16_t *dz, *dzt, *wt, *ht;  // generic
  uint16_t *dz2, *ht2;           // direct-to-LDS (pair of tiles)
  float* hpart;
};

size_t bwd_scratch_bytes(int64_t tr, int64_t h, int64_t vpad) {
  const size_t tpad = align_up(static_cast<size_t>(tr), 64), V = static_cast<size_t>(vpad), H = static_cast<size_t>(h);
  const size_t part = align_up(static_cast<size_t>(kSplitK) * tr * H * 4, 256);
  const size_t generic = align_up(tpad * V * 2, 256) * 2 + align_up(H * V * 2, 256) + align_up(H * tpad * 2, 256);
  const size_t fast = align_up(2 * tpad * V * 2, 256) + align_up(2 * tpad * H * 2, 256);
  return (generic > fast ? generic : fast) + part;
}

BwdBuffers bwd_buffers(char* base, int64_t tr, int64_t h, int64_t vpad) {
  const size_t tpad = align_up(static_cast<size_t>(tr), 64), V = static_cast<size_t>(vpad), H = static_cast<size_t>(h);
  BwdBuffers b;
  size_t off = 0;
  b.dz = b.dz2 = reinterpret_cast<uint16_t*>(base);
  off = align_up(tpad * V * 2, 256);
  b.dzt = reinterpret_cast<uint16_t*>(base + off);
  off += align_up(tpad * V * 2, 256);
  b.wt = reinterpret_cast<uint16_t*>(base + off);
  off += align_up(H * V * 2, 256);
  b.ht = reinterpret_cast<uint16_t*>(base + off);
  off += align_up(H * tpad * 2, 256);
  b.ht2 = reinterpret_cast<uint16_t*>(base + align_up(2 * tpad * V * 2, 256));
  const size_t fast = align_up(2 * tpad * V * 2, 256) + align_up(2 * tpad * H * 2, 256);
  b.hpart = reinterpret_cast<float*>(base + (off > fast ? off : fast));
  return b;
}

// One dispatch covers at most 2^32 - 1 work-items per grid dimension.  True
// when every launch of the call (fast or generic tiles) stays within that.
bool lmhead_launches_fit(int64_t T, int64_t h, int64_t V, int64_t tile_rows, int backward) {
  if (T <= 0) return true;
  auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  const int64_t tr = tile_rows < T ? tile_rows : T;
  int64_t m = 0;
  auto add = [&](int64_t blocks, int64_t threads) {
    if (blocks * threads > m) m = blocks * threads;
  };
  if (backward == 0) {
    const int64_t g = cdiv(T, tr) < kFwdTilesPerLaunch ? cdiv(T, tr) : kFwdTilesPerLaunch;
    add((cdiv(V, FwdDtlCfg::BM) * cdiv(tr * g, FwdDtlCfg::BN) + 7) / 8 * 8, FwdDtlCfg::NT);
    add((cdiv(V, FwdCfg::BM) * cdiv(tr, FwdCfg::BN) + 7) / 8 * 8, FwdCfg::NT);
    add(cdiv(tr * g, 4), 256);
  } else if (backward == 2) {
    const int64_t ch = tr < kKLChunk ? tr : kKLChunk;
    add(cdiv(V, KLCfg::BM) * cdiv(ch, KLCfg::BN), KLCfg::NT);
    add(cdiv(V, FwdCfg::BM) * cdiv(ch, FwdCfg::BN), FwdCfg::NT);
    add(cdiv(ch, 4), 256);
  } else {
    add(cdiv(V, BwdDtlCfg::BM) * cdiv(tr, BwdDtlCfg::BN), BwdDtlCfg::NT);
    add(cdiv(V, BwdCfg::BM) * cdiv(tr, BwdCfg::BN), BwdCfg::NT);
    add(cdiv(tr, DenseDtlCfg::BM) * cdiv(h, DenseDtlCfg::BN) * kSplitK, DenseDtlCfg::NT);
    add(cdiv(tr, BwdCfg::BM) * cdiv(h, BwdCfg::BN), BwdCfg::NT);
    add(cdiv(V, DenseDtlCfg::BM) * cdiv(h, DenseDtlCfg::BN), DenseDtlCfg::NT);
    add(cdiv(V, BwdCfg::BM) * cdiv(h, BwdCfg::BN), BwdCfg::NT);
    add(cdiv(V, 64) + 1, 256);   // W^T transpose, x dimension
    add(cdiv(tr, 64) + 1, 256);  // hidden-tile transpose, x dimension
  }
  return m <= 0xffffffffll;
}

bool lmhead_workspace_layout(int64_t T, int64_t h, int64_t V, int64_t tile_rows, int backward,
                             LMHeadWorkspace* w) {
  if (T < 0 || h <= 0 || V <= 0 || tile_rows <= 0) return false;
  if (T > 0x7fffffff || V > (int64_t(1) << 30) || h > (int64_t(1) << 30)) return false;
  const int64_t tr = tile_rows < (T > 0 ? T : 1) ? tile_rows : (T > 0 ? T : 1);
  const int bm_min = FwdCfg::BM < FwdDtlCfg::BM ? FwdCfg::BM : FwdDtlCfg::BM;
  w->n_vblocks = static_cast<int>((V + bm_min - 1) / bm_min);  // enough partials for either forward tile
  w->vpad = static_cast<int64_t>(align_up(static_cast<size_t>(V), 64));
  size_t off = 0;
  w->idx_off = off;
  off = align_up(off + static_cast<size_t>(T > 0 ? T : 1) * 4, 256);
  w->count_off = off;
  off += 256;
  w->part_off = w->zy_off = w->dz_off = 0;
  w->tbuf_off = 0;
  if (backward == 0 || backward == 2) {
    // log-prob forward: 3 floats per partial state, up to kMaxTargets target logits per row;
    // KL forward: 5 floats per dual state, the student and teacher target logits per row
    // (the KL forward runs chunks of at most kKLChunk rows; the fast log-prob
    // forward launches up to kFwdTilesPerLaunch tiles at once, with fewer
    // vocab blocks per row)
    const int fields = backward == 0 ? 3 : 5;
    const int per_row = backward == 0 ? kMaxTargets : 2;
    const int64_t prow = backward == 2 && tr > kKLChunk ? kKLChunk : tr;
    size_t states = static_cast<size_t>(prow) * w->n_vblocks;
    size_t zrows = static_cast<size_t>(prow);
    if (backward == 0) {
      const int64_t tiles = (T + tr - 1) / tr;
      const int64_t g = tiles < kFwdTilesPerLaunch ? (tiles > 0 ? tiles : 1) : kFwdTilesPerLaunch;
      const size_t fast = static_cast<size_t>(g * tr) * static_cast<size_t>((V + FwdDtlCfg::BM - 1) / FwdDtlCfg::BM);
      if (fast > states) states = fast;
      zrows = static_cast<size_t>(g * tr);
    }
    w->part_off = off;
    off = align_up(off + states * fields * 4, 256);
    w->zy_off = off;
    off = align_up(off + zrows * per_row * 4, 256);
  } else {  // backward == 1 or 3
    // generic tiles: dZ [tpad x vpad], dZ^T [vpad x tpad], W^T [h x vpad], H_tile^T [h x tpad];
    // direct-to-LDS tiles: dZ of two tiles [2 tpad x vpad], their hidden rows [2 tpad x h];
    // both: the split-K partials of dHidden [kSplitK x tr x h] fp32 (see bwd_buffers)
    w->dz_off = off;
    off += bwd_scratch_bytes(tr, h, w->vpad);
  }
  if (backward >= 2) {
    // teacher logits of one chunk: [vocab block][row block][BM x BN] floats
    const int64_t chunk = tr < kKLChunk ? tr : kKLChunk;
    const int64_t nvb = (V + KLCfg::BM - 1) / KLCfg::BM, nnb = (chunk + KLCfg::BN - 1) / KLCfg::BN;
    w->tbuf_off = off;
    off = align_up(off + static_cast<size_t>(nvb * nnb) * KLCfg::BM * KLCfg::BN * 4, 256);
  }
  w->total = off;
  return true;
}

// ---------------------------------------------------------------------------
// scored-row compaction
// ---------------------------------------------------------------------------

// Per-row outputs that unscored rows get as zeros: up to 6 arrays of
// width[i] floats per row (null pointers skipped).
struct ZeroOuts {
  float* p[6];
  int width[6];
};

static ZeroOuts zero_outs(float* a = nullptr, int wa = 1, float* b = nullptr, float* c = nullptr, float* d = nullptr,
                   float* e = nullptr, float* f = nullptr) {
  return ZeroOuts{{a, b, c, d, e, f}, {wa, 1, 1, 1, 1, 1}};
}

__global__ void __launch_bounds__(1024) k_compact(const uint8_t* __restrict__ mask, int64_t T, int* __restrict__ idx,
                                                  int* __restrict__ count, ZeroOuts z) {
  // Rounds of 1024 x R rows; thread t owns rows [base + R t, base + R t + R),
  // so the workgroup reads each round's mask bytes together and an exclusive
  // scan of the per-thread counts (wave shuffles, then the 16 wave totals)
  // gives ascending positions.
  constexpr int R = 16;
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int total = 0;  // scored rows before this round (uniform)
  for (int64_t base = 0; base < T; base += 1024 * R) {
    const int64_t b = base + static_cast<int64_t>(tid) * R;
    unsigned bits = 0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int64_t i = b + j;
      if (i < T && (mask == nullptr || mask[i] != 0)) bits |= 1u << j;
    }
    const int c = __popc(bits);
    int incl = c;  // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0, round_total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int v = wsum[w];
      before += w < wave ? v : 0;
      round_total += v;
    }
    int pos = total + before + incl - c;
    for (int j = 0; j < R; ++j) {
      const int64_t i = b + j;
      if (i >= T) break;
      if ((bits >> j) & 1u) {
        idx[pos++] = static_cast<int>(i);
      } else {
#pragma unroll
        for (int q = 0; q < 6; ++q)
          if (z.p[q])
            for (int k = 0; k < z.width[q]; ++k) z.p[q][i * z.width[q] + k] = 0.f;
      }
    }
    total += round_total;
    __syncthreads();  // wsum is rewritten by the next round
  }
  if (tid == 0) *count = total;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------

struct FwdArgs {
  const uint16_t* weight;
  int64_t ld_w;
  const uint16_t* hidden;
  int64_t ld_h;
  int h, V;
  const int* idx;
  const int* count;
  const int64_t* targets;  // [T x K]
  int K;
  float c;
  int64_t tile_base;  // first compacted row of the launch
  int tile_rows;      // rows of the launch (its tiles together)
  int n_vb, n_nb;     // vocab blocks, row blocks of the launch
  float* part;        // [tile_rows][n_vb][3]
  float* zy;          // [tile_rows][K]
  int clocks;         // record per-workgroup clock samples (timing mode 2)
};

// Block -> (vocab block, row block) of a launch.  The fast forward blocks the
// rows of all the tiles of its launch as one sequence (row blocks may straddle
// tiles; every row's result is the same either way), so only the launch's last
// row block is partly filled.  The grid is sized on the host for every row of
// the launch's tiles, but only the row blocks holding scored rows (the count
// is on the device) are mapped: blocks 0 .. n_vb * live - 1 take them and the
// rest exit at once, so empty row blocks take no place in the walk below.
// Logical order: group of kGroupV vocab blocks -> row block -> vocab block
// within the group, and each XCD (hardware puts workgroup b on XCD b % 8)
// walks one contiguous range of that order: a group's weight rows serve every
// row of the launch back to back while they are still cached (the weight
// comes from HBM once per launch, not once per tile), and the 32 workgroups
// an XCD runs at once cover 4 vocab blocks x 8 row blocks, which share their
// strips in its L2.  False for blocks without work; `rows` = scored rows of
// the launch.
template <int BN>
__device__ __forceinline__ bool fwd_block(const FwdArgs& a, int& vb, int& nb, int& rows) {
  const int64_t rem = static_cast<int64_t>(*a.count) - a.tile_base;
  rows = static_cast<int>(rem < a.tile_rows ? rem : a.tile_rows);
  if (rows <= 0) return false;
  const int n_nb = (rows + BN - 1) / BN;  // live row blocks (<= a.n_nb)
  const int live = a.n_vb * n_nb;
  const int b = static_cast<int>(blockIdx.x);
  if (b >= live) return false;
  const int L = xcd_remap(b, live);
  constexpr int G = kGroupV;
  const int full = a.n_vb / G;
  const int span = G * n_nb;  // blocks of a full group
  const int g = L / span;
  int gsz = G, w = L - g * span, v0 = g * G;
  if (g >= full) {  // the last, smaller group
    gsz = a.n_vb - full * G;
    w = L - full * span;
    v0 = full * G;
  }
  nb = w / gsz;
  vb = v0 + w % gsz;
  return true;
}

// Forward epilogue shared by both GEMM mainloops: per token column, fold the
// block's vocab rows into one (mc, s, a) state, pick up the target logit if
// its column lies in this block, and write one partial per (row, vocab block).
template <class C>
__device__ __forceinline__ void fwd_epilogue(const FwdArgs& a, f32x16_t (&acc)[C::MI][C::NI], int vb, int n0, int rows,
                                             uint16_t* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WGM, wn = wave / C::WGM;
  const int vwave = vb * C::BM + wm * C::WTM;  // first vocab row of this wave
  const int half = lane >> 5;
  Stat* sm = reinterpret_cast<Stat*>(lds);  // [WGM][BN] states, reused after the K loop
  const float c = a.c;
  const bool full_block = (vb + 1) * C::BM <= a.V;  // uniform
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int nl = wn * C::WTN + ni * 32 + (lane & 31);
    const int r = n0 + nl;  // row within the tile
    const bool valid_row = r < rows;
    const int64_t row = valid_row ? a.idx[a.tile_base + r] : 0;
    Stat st = stat_empty();
    if (full_block) {
      // every vocab row of this block exists: one fold over all of this
      // lane's values of the row (one max, no rebase)
      float x[C::MI * 16];
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i) x[mi * 16 + i] = acc[mi][ni][i];
      stat_push<false, C::MI * 16, 16>(st, x, c);
    } else {
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi) {
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = vwave + mi * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          // rows past V hold zeros from the GEMM: probability 0 (-inf with the clamped fold)
          x[i] = (v < a.V) ? acc[mi][ni][i] : -INFINITY;
        }
        stat_push<true, 16, 16>(st, x, c);
      }
    }
    // target logits whose column lies in this wave's vocab rows
    for (int k = 0; valid_row && k < a.K; ++k) {
      const int64_t yrel = a.targets[row * a.K + k] - vwave;
      if (yrel >= 0 && yrel < C::WTM) {
        float zsel = 0.f;
        bool found = false;
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int vr = mi * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            if (yrel == vr) {
              zsel = acc[mi][ni][i];
              found = true;
            }
          }
        if (found) a.zy[static_cast<int64_t>(r) * a.K + k] = zsel;
      }
    }
    Stat o;
    o.mc = __shfl_xor(st.mc, 32, 64);
    o.s = __shfl_xor(st.s, 32, 64);
    o.a = __shfl_xor(st.a, 32, 64);
    st = stat_merge(st, o);
    if (lane < 32) sm[wm * C::BN + nl] = st;
    __builtin_amdgcn_sched_barrier(0);  // one token column at a time: bounds the live registers
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni) {
      const int nl = wn * C::WTN + ni * 32 + lane;
      const int r = n0 + nl;
      if (r < rows) {
        Stat st = sm[nl];
#pragma unroll
        for (int k = 1; k < C::WGM; ++k) st = stat_merge(st, sm[k * C::BN + nl]);
        float* p = a.part + (static_cast<int64_t>(r) * a.n_vb + vb) * 3;
        p[0] = st.mc;
        p[1] = st.s;
        p[2] = st.a;
      }
    }
  }
}

// Generic forward tile (any h % 8 == 0): register-staged, zero-filled loads.
template <class C>
__global__ void __launch_bounds__(C::NT) k_fwd_tile(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  int vb, nb, rows;
  if (!fwd_block<C::BN>(a, vb, nb, rows)) return;
  const int n0 = nb * C::BN;
  const int v0 = vb * C::BM;
  GemmOperands op;
  op.a = a.weight + static_cast<int64_t>(v0) * a.ld_w;
  op.lda = a.ld_w;
  op.M = a.V - v0;
  op.b = a.hidden;
  op.ldb = a.ld_h;
  op.b_rows = a.idx + a.tile_base + n0;
  op.N = rows - n0;
  op.K = a.h;
  f32x16_t acc[C::MI][C::NI];
  gemm_tile<C>(op, 0, 0, lds, acc);
  fwd_epilogue<C>(a, acc, vb, n0, rows, lds);
}

// Clock samples of the fast forward (timing mode 2, observability only): for
// workgroup b < kClockSamples of the last such launch, the deltas of the
// shader-clock counter and of the fixed-frequency counter over its run.
constexpr int kClockSamples = 65536;
__device__ unsigned long long g_fwd_clocks[2 * kClockSamples];
int64_t g_fwd_clock_blocks = 0;  // workgroups of the last sampled launch (host)

hipError_t read_fwd_clocks(unsigned long long* pairs, int64_t* n) {
  const int64_t m = g_fwd_clock_blocks < kClockSamples ? g_fwd_clock_blocks : kClockSamples;
  if (*n > m) *n = m;
  if (*n <= 0) {
    *n = 0;
    return hipSuccess;
  }
  return hipMemcpyFromSymbol(pairs, HIP_SYMBOL(g_fwd_clocks), sizeof(unsigned long long) * 2 * (*n));
}

// Fast forward tile (h % 64 == 0): direct-to-LDS loads, 256 (vocab) x 320
// (rows) block.
template <class C>
__global__ void __launch_bounds__(C::NT, LP_FWD_MIN_WAVES) k_fwd_tile_dtl(FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_ELEMS];
  // clock samples: the start values go to memory and are read back at the
  // end (volatile), so nothing stays live in registers across the K loop
  volatile unsigned long long* clk = g_fwd_clocks + 2 * blockIdx.x;
  const bool sample = a.clocks && threadIdx.x == 0 && blockIdx.x < kClockSamples;
  if (sample) {
    clk[0] = __builtin_amdgcn_s_memtime();
    clk[1] = __builtin_amdgcn_s_memrealtime();
  }
  int vb, nb, rows;
  if (!fwd_block<C::BN>(a, vb, nb, rows)) {
    if (sample) clk[1] = 0;  // no work: a zero fixed-clock delta, skipped by the reader
    return;
  }
  const int n0 = nb * C::BN;
  const int v0 = vb * C::BM;
  f32x16_t acc[C::MI][C::NI];
  gemm_tile_dtl<C>(a.weight + static_cast<int64_t>(v0) * a.ld_w, a.ld_w, a.V - v0, a.hidden, a.ld_h,
                   a.idx + a.tile_base + n0, rows - n0, a.h, lds, acc);
  fwd_epilogue<C>(a, acc, vb, n0, rows, lds);
  if (sample) {
    clk[0] = __builtin_amdgcn_s_memtime() - clk[0];
    clk[1] = __builtin_amdgcn_s_memrealtime() - clk[1];
  }
}

struct MergeArgs {
  const float* part;
  const float* zy;
  int n_vb;
  const int* idx;
  const int* count;
  const int64_t* targets;  // [T x K]
  int K;
  int V;
  float c;
  int64_t tile_base;
  int tile_rows;   // rows of all the launch's tiles
  float* logprob;  // [T x K]
  float* entropy;
  float* lse;
};

__global__ void __launch_bounds__(256) k_fwd_merge(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int count = *a.count;
  const int64_t rem = static_cast<int64_t>(count) - a.tile_base;
  const int rows = static_cast<int>(rem < a.tile_rows ? rem : a.tile_rows);
  if (r >= rows) return;
  const float* p = a.part + static_cast<int64_t>(r) * a.n_vb * 3;
  Stat st = stat_empty();
  for (int vb = lane; vb < a.n_vb; vb += 64) st = stat_merge(st, Stat{p[vb * 3], p[vb * 3 + 1], p[vb * 3 + 2]});
  st = stat_wave_allreduce(st);
  const int64_t row = a.idx[a.tile_base + r];
  const float l2s = log2f(st.s);
  for (int k = lane; k < a.K; k += 64) {
    const int64_t y = a.targets[row * a.K + k];
    float lp = __builtin_nanf("");
    if (y >= 0 && y < a.V) lp = (fmaf(a.zy[static_cast<int64_t>(r) * a.K + k], a.c, -st.mc) - l2s) * kLn2;
    a.logprob[row * a.K + k] = lp;
  }
  if (lane == 0) {
    if (a.entropy) a.entropy[row] = (l2s - st.a / st.s) * kLn2;
    if (a.lse) a.lse[row] = (st.mc + l2s) * kLn2;
  }
}

hipError_t launch_lmhead_forward(const LMHeadShape& sh, float* logprob, float* entropy, float* lse, char* ws,
                                 const LMHeadWorkspace& w, hipStream_t s) {
  int* idx = reinterpret_cast<int*>(ws + w.idx_off);
  int* count = reinterpret_cast<int*>(ws + w.count_off);
  float* part = reinterpret_cast<float*>(ws + w.part_off);
  float* zy = reinterpret_cast<float*>(ws + w.zy_off);
  {
    TimedLaunch tl("k_compact", s);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, s, sh.mask, sh.T, idx, count,
                       zero_outs(logprob, sh.K, entropy, lse));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tr = sh.tile_rows < sh.T ? sh.tile_rows : sh.T;
  // K multiple of 64: direct-to-LDS 256 x 256 tiles, several row tiles per
  // launch; otherwise the generic tile, one row tile per launch
  const bool fast = lmhead_fast_path(sh);
  const int bm = fast ? FwdDtlCfg::BM : FwdCfg::BM;
  const int bn = fast ? FwdDtlCfg::BN : FwdCfg::BN;
  const int n_vb = (sh.V + bm - 1) / bm;
  const int64_t group = fast ? kFwdTilesPerLaunch : 1;
  for (int64_t base = 0; base < sh.T; base += group * tr) {
    const int64_t left = (sh.T - base + tr - 1) / tr;
    const int ntile = static_cast<int>(left < group ? left : group);
    // the launch's ntile * tr rows in row blocks of bn, vocab blocks of bm
    const int n_nb = static_cast<int>((tr * ntile + bn - 1) / bn);
    const int grid_blocks = n_vb * n_nb;  // blocks past the scored rows' blocks exit at once
    FwdArgs a;
    a.weight = sh.weight;
    a.ld_w = sh.ld_w;
    a.hidden = sh.hidden;
    a.ld_h = sh.ld_h;
    a.h = sh.h;
    a.V = sh.V;
    a.idx = idx;
    a.count = count;
    a.targets = sh.targets;
    a.K = sh.K;
    a.c = sh.c;
    a.tile_base = base;
    a.tile_rows = static_cast<int>(tr * ntile);
    a.n_vb = n_vb;
    a.n_nb = n_nb;
    a.part = part;
    a.zy = zy;
    a.clocks = fast && timing_clocks_on() ? 1 : 0;
    if (a.clocks) g_fwd_clock_blocks = grid_blocks;
    {
      TimedLaunch tl("k_fwd_tile", s);
      const dim3 grid(static_cast<unsigned>(grid_blocks));
      if (fast)
        hipLaunchKernelGGL(k_fwd_tile_dtl<FwdDtlCfg>, grid, dim3(FwdDtlCfg::NT), 0, s, a);
      else
        hipLaunchKernelGGL(k_fwd_tile<FwdCfg>, grid, dim3(FwdCfg::NT), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    MergeArgs m;
    m.part = part;
    m.zy = zy;
    m.n_vb = n_vb;
    m.idx = idx;
    m.count = count;
    m.targets = sh.targets;
    m.K = sh.K;
    m.V = sh.V;
    m.c = sh.c;
    m.tile_base = base;
    m.tile_rows = static_cast<int>(tr * ntile);
    m.logprob = logprob;
    m.entropy = entropy;
    m.lse = lse;
    {
      TimedLaunch tl("k_fwd_merge", s);
      hipLaunchKernelGGL(k_fwd_merge, dim3(static_cast<unsigned>((tr * ntile + 3) / 4)), dim3(256), 0, s, m);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------

// Tiled transpose of bf16 rows: dst[c][r] = src_row(r)[c] for r < nr, c < nc;
// zero for r in [nr, nr_pad), c < nc.  src_row(r) = src + rows[r] * ld (or r * ld).
__global__ void __launch_bounds__(256) k_transpose_bf16(const uint16_t* __restrict__ src, int64_t ld,
                                                        const int* __restrict__ rows, const int* __restrict__ count,
                                                        int64_t row_base, int nr_static, int nr_cap, int nr_pad,
                                                        int nc, uint16_t* __restrict__ dst, int64_t ldd) {
  __shared__ uint16_t t[64][65];
  int nr = nr_static;
  if (count) {
    const int64_t rem = static_cast<int64_t>(*count) - row_base;
    nr = static_cast<int>(rem < nr_cap ? (rem > 0 ? rem : 0) : nr_cap);
  }
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  if (r0 >= nr_pad) return;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int r = r0 + k, cc = c0 + tx;
    uint16_t v = 0;
    if (r < nr && cc < nc) {
      const int64_t sr = rows ? static_cast<int64_t>(rows[row_base + r]) : static_cast<int64_t>(r);
      v = src[sr * ld + cc];
    }
    t[k][tx] = v;
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int cc = c0 + k, r = r0 + tx;
    if (cc < nc && r < nr_pad) dst[static_cast<int64_t>(cc) * ldd + r] = t[tx][k];
  }
}

__global__ void __launch_bounds__(256) k_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  {
    TimedLaunch tl("k_zero_f32", s);
    hipLaunchKernelGGL(k_zero_f32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n);
  }
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) k_zero_unscored_rows(const uint8_t* __restrict__ mask, int64_t T, int h,
                                                            float* __restrict__ out) {
  for (int64_t row = blockIdx.x; row < T; row += gridDim.x) {
    if (mask != nullptr && mask[row] == 0) {
      float* p = out + row * h;
      for (int j = threadIdx.x; j < h; j += 256) p[j] = 0.f;
    }
  }
}

struct DzArgs {
  const uint16_t* weight;
  int64_t ld_w;
  const uint16_t* hidden;
  int64_t ld_h;
  int h, V;
  int64_t vpad;
  const int* idx;
  const int* count;
  const int64_t* targets;  // [T x K]
  int K;
  const float* lse;
  const float* entropy;
  const float* g_lp;  // [T x K]
  const float* g_H;
  float c, inv_tau;
  int64_t tile_base;
  int tile_rows;
  int64_t tpad;
  int n_vb, n_nb;
  uint16_t* dz;   // [tpad][vpad]
  uint16_t* dzt;  // [vpad][tpad] or nullptr
};

// Four consecutive vocab columns vq..vq+3 of tile row r, packed bf16 in pk
// (generic tiles): four 2-byte stores into dZ^T [vocab][row] ...
__device__ __forceinline__ void dzt_store4(uint16_t* dzt, int64_t tpad, int r, int vq, uint2 pk) {
  dzt[static_cast<int64_t>(vq) * tpad + r] = static_cast<uint16_t>(pk.x);
  dzt[static_cast<int64_t>(vq + 1) * tpad + r] = static_cast<uint16_t>(pk.x >> 16);
  dzt[static_cast<int64_t>(vq + 2) * tpad + r] = static_cast<uint16_t>(pk.y);
  dzt[static_cast<int64_t>(vq + 3) * tpad + r] = static_cast<uint16_t>(pk.y >> 16);
}

// ... and one 8-byte store into dZ [row][vocab] (plus dZ^T if requested).
__device__ __forceinline__ void dz_store4(uint16_t* dz, uint16_t* dzt, int64_t vpad, int64_t tpad, int r, int vq,
                                          uint2 pk) {
  *reinterpret_cast<uint2*>(dz + static_cast<int64_t>(r) * vpad + vq) = pk;
  if (dzt) dzt_store4(dzt, tpad, r, vq, pk);
}

// Staged dZ rows: the fast kernels first write their tile of dZ [rows][vocab]
// to LDS with a row pitch of BM + 4 elements (consecutive tile rows then fall
// in different banks for the 8-byte writes of one MFMA column), then copy
// whole rows out with 16-byte stores, so every 32 lanes write 512 contiguous
// bytes instead of 32 scattered 8-byte pieces.
template <class C>
struct DzStage {
  static constexpr int P = C::BM + 4;
  static constexpr int ELEMS = C::BN * P;
};

__device__ __forceinline__ void dz_stage4(uint16_t* lds, int pitch, int r_local, int v_local, uint2 pk) {
  *reinterpret_cast<uint2*>(lds + r_local * pitch + v_local) = pk;
}

// Copies the staged rows [0, nrow) of the tile (vocab columns v0 + [0, BM),
// clipped to vpad) to dZ [row][vocab].  Needs a barrier before (all staged
// writes done); LDS is not reused afterwards.
template <class C>
__device__ __forceinline__ void dz_flush_rows(const uint16_t* lds, uint16_t* dz, int64_t vpad, int v0, int n0,
                                              int nrow) {
  constexpr int P = DzStage<C>::P;
  constexpr int NCH = C::BM / 8;  // 16-byte chunks per row
  for (int idx = threadIdx.x; idx < nrow * NCH; idx += C::NT) {
    const int r = idx / NCH, ch = idx % NCH;
    const int v = v0 + ch * 8;
    if (v >= vpad) continue;
    const uint2 lo = *reinterpret_cast<const uint2*>(lds + r * P + ch * 8);
    const uint2 hi = *reinterpret_cast<const uint2*>(lds + r * P + ch * 8 + 4);
    *reinterpret_cast<uint4*>(dz + static_cast<int64_t>(n0 + r) * vpad + v) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
}

// Copies the staged rows [0, nrow) (nrow a multiple of 64) to dZ^T
// [vocab][row]: each thread gathers 8 consecutive rows of one vocab column
// from LDS and writes them with one 16-byte store; the 64 lanes of a wave
// take 8 row octets x 8 columns, so each store instruction fills 8 whole
// 128-byte lines.  Needs the same barrier as dz_flush_rows.
template <class C>
__device__ __forceinline__ void dzt_flush_cols(const uint16_t* lds, uint16_t* dzt, int64_t tpad, int64_t vpad, int v0,
                                               int n0, int nrow) {
  constexpr int P = DzStage<C>::P;
  constexpr int NVO = C::BM / 8;  // vocab octets
  const int nitems = (nrow / 8) * C::BM;
  for (int idx = threadIdx.x; idx < nitems; idx += C::NT) {
    const int blk = idx / 64, w = idx % 64;
    const int g = (blk / NVO) * 8 + (w & 7);  // row octet
    const int vl = (blk % NVO) * 8 + (w >> 3);
    const int64_t v = v0 + vl;
    if (v >= vpad) continue;
    uint32_t q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      q[j] = static_cast<uint32_t>(lds[(g * 8 + 2 * j) * P + vl]) |
             (static_cast<uint32_t>(lds[(g * 8 + 2 * j + 1) * P + vl]) << 16);
    *reinterpret_cast<uint4*>(dzt + v * tpad + n0 + g * 8) = make_uint4(q[0], q[1], q[2], q[3]);
  }
}

// dL/dlogits epilogue: for tile rows r < rowsK (the K span of the
// weight-gradient GEMM; rows past the tile's valid rows get 0) and vocab
// columns v < vpad (0 past V), writes bf16 dZ[r][v] and, if requested, dZ^T[v][r].
template <class C, bool STAGED>
__device__ __forceinline__ void dz_epilogue(const DzArgs& a, f32x16_t (&acc)[C::MI][C::NI], int v0, int n0, int rows,
                                            int rowsK, uint16_t* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WGM, wn = wave / C::WGM;
  const int vlane = v0 + wm * C::WTM + 4 * (lane >> 5);
  const bool full_block = v0 + C::BM <= a.V;  // uniform: every vocab column of the block exists
  const float it = a.inv_tau;
  // dZ = it * [sum_k g_k onehot_k - p (gsum + gH (z it - mu))] = it * sum_k g_k onehot_k - p (A + B z).
  // The per-row constants of all token columns, as two batches of independent
  // loads (row indices, then the rows' values) rather than one dependent pair
  // per column; row 0 stands in for columns past the valid rows.
  int64_t row_n[C::NI], y0_n[C::NI];
  float l2_n[C::NI], A_n[C::NI], B_n[C::NI], g0_n[C::NI];
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int r = n0 + wn * C::WTN + ni * 32 + (lane & 31);
    row_n[ni] = r < rows ? a.idx[a.tile_base + r] : 0;
  }
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int64_t row = row_n[ni];
    const float L = a.lse[row];
    const float mu = L - a.entropy[row];
    y0_n[ni] = a.targets[row * a.K];
    g0_n[ni] = a.g_lp[row * a.K];
    float gsum = g0_n[ni];
    for (int k = 1; k < a.K; ++k) gsum += a.g_lp[row * a.K + k];
    const float gh = a.g_H ? a.g_H[row] : 0.f;
    l2_n[ni] = L * kLog2eF;
    A_n[ni] = it * fmaf(-gh, mu, gsum);
    B_n[ni] = it * it * gh;
  }
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int r = n0 + wn * C::WTN + ni * 32 + (lane & 31);
    if (r >= rowsK) continue;
    const bool valid = r < rows;
    const int64_t row = row_n[ni], y0 = valid ? y0_n[ni] : -1;
    const float l2 = valid ? l2_n[ni] : 0.f, A = valid ? A_n[ni] : 0.f, B = valid ? B_n[ni] : 0.f;
    const float g0 = valid ? g0_n[ni] : 0.f;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int vq = vlane + mi * 32 + 8 * q;
        float d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float z = acc[mi][ni][q * 4 + j];
          const float p = fast_exp2(fmaf(z, a.c, -l2));
          d[j] = valid ? -p * fmaf(B, z, A) : 0.f;
          if (!full_block && vq + j >= a.V) d[j] = 0.f;
        }
        if (valid) {
          // the row's targets inside these four columns (usually none)
          const int64_t y0rel = y0 - vq;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (y0rel == j) d[j] += it * g0;
          for (int k = 1; k < a.K; ++k) {
            const int64_t yrel = a.targets[row * a.K + k] - vq;
            if (yrel >= 0 && yrel < 4) {
              const float gk = it * a.g_lp[row * a.K + k];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (yrel == j) d[j] += gk;
            }
          }
        }
        const uint2 pk = pack_bf16x4(d);
        if (STAGED)
          dz_stage4(lds, DzStage<C>::P, r - n0, vq - v0, pk);
        else if (vq < a.vpad)
          dz_store4(a.dz, a.dzt, a.vpad, a.tpad, r, vq, pk);
      }
  }
  if (STAGED) {
    __syncthreads();
    const int nrow = (rowsK - n0) < C::BN ? (rowsK - n0) : C::BN;
    dz_flush_rows<C>(lds, a.dz, a.vpad, v0, n0, nrow);
    if (a.dzt) dzt_flush_cols<C>(lds, a.dzt, a.tpad, a.vpad, v0, n0, nrow);
  }
}

// Generic recompute tile (any h % 8 == 0).
template <class C>
__global__ void __launch_bounds__(C::NT) k_bwd_dz(DzArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  int vb, nb;
  tile_coords(xcd_remap(blockIdx.x, a.n_vb * a.n_nb), a.n_vb, a.n_nb, vb, nb);
  const int count = *a.count;
  const int64_t rem = static_cast<int64_t>(count) - a.tile_base;
  const int rows = static_cast<int>(rem < a.tile_rows ? rem : a.tile_rows);
  const int rowsK = (rows + 7) & ~7;
  const int n0 = nb * C::BN;
  if (rows <= 0 || n0 >= rowsK) return;
  const int v0 = vb * C::BM;
  GemmOperands op;
  op.a = a.weight + static_cast<int64_t>(v0) * a.ld_w;
  op.lda = a.ld_w;
  op.M = a.V - v0;
  op.b = a.hidden;
  op.ldb = a.ld_h;
  op.b_rows = a.idx + a.tile_base + n0;
  op.N = rows - n0;
  op.K = a.h;
  f32x16_t acc[C::MI][C::NI];
  gemm_tile<C>(op, 0, 0, lds, acc);
  dz_epilogue<C, false>(a, acc, v0, n0, rows, rowsK, lds);
}

// Fast recompute tile (h % 64 == 0): the forward's direct-to-LDS mainloop.
// Rows up to the next multiple of 64 are written (zeros past the valid rows)
// because the fast weight-gradient GEMM takes K in steps of 64.
template <class C>
__global__ void __launch_bounds__(C::NT) k_bwd_dz_dtl(DzArgs a) {
  constexpr int kLds = C::LDS_ELEMS > DzStage<C>::ELEMS ? C::LDS_ELEMS : DzStage<C>::ELEMS;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kLds];
  int vb, nb;
  tile_coords(xcd_remap(blockIdx.x, a.n_vb * a.n_nb), a.n_vb, a.n_nb, vb, nb);
  const int count = *a.count;
  const int64_t rem = static_cast<int64_t>(count) - a.tile_base;
  const int rows = static_cast<int>(rem < a.tile_rows ? rem : a.tile_rows);
  const int rowsK = (rows + 63) & ~63;
  const int n0 = nb * C::BN;
  if (rows <= 0 || n0 >= rowsK) return;
  const int v0 = vb * C::BM;
  f32x16_t acc[C::MI][C::NI];
  gemm_tile_dtl<C>(a.weight + static_cast<int64_t>(v0) * a.ld_w, a.ld_w, a.V - v0, a.hidden, a.ld_h,
                   a.idx + a.tile_base + n0, rows - n0, a.h, lds, acc);
  dz_epilogue<C, true>(a, acc, v0, n0, rows, rowsK, lds);
}

// Fast gradient GEMMs (K multiple of 64) on the dZ buffer [rows][vpad] as
// written by the dZ kernels:
//   dHidden: A = dZ (K-contiguous, K = vpad), B = W (K-major: row v of the
//            weight is K index v; rows past V are clamped, their dZ columns
//            are 0), K split into `splits` ranges; each split writes an fp32
//            partial [rows x h] that k_splitk_reduce sums in a fixed order.
//   dW:      A = dZ (K-major, M = vocab), B = the tiles' hidden rows [rows][h]
//            (K-major), K = the rows of one or two consecutive tiles (the
//            second tile's rows start at row tpad); dW is written (first
//            launch) or accumulated.
struct DenseGemmArgs {
  const uint16_t* a;
  int64_t lda;
  int M;              // if m_from_count: the tile's valid rows instead
  const uint16_t* b;
  int64_t ldb;
  int N;
  int K;              // if k_from_count: the tiles' rows, each tile rounded up to 64
  int kvalid_b;       // K-major B: rows of B that exist
  const int* count;
  int64_t tile_base;
  int tile_rows;
  int64_t tpad;       // k_from_count: row offset of the second tile
  int ntiles;         // k_from_count: tiles in this launch (1 or 2)
  int m_from_count, k_from_count;
  int splits;         // K ranges (blockIdx spans n_mb * n_nb * splits)
  int ksplit;         // K per split (multiple of 64)
  float* out;         // dW [M x ldo] or partials [splits][tile_rows][ldo]
  int64_t ldo;
  int accumulate;
  int n_mb, n_nb;
};

// Valid rows of tile `t` of a launch (device count).
__device__ __forceinline__ int tile_rows_of(const int* count, int64_t base, int tile_rows, int t) {
  const int64_t rem = static_cast<int64_t>(*count) - base - static_cast<int64_t>(t) * tile_rows;
  return static_cast<int>(rem < tile_rows ? (rem > 0 ? rem : 0) : tile_rows);
}

// Row blocks per group in the walk of the gradient GEMMs (tile_coords): the
// hidden-gradient GEMM's rows are the tile's rows, the weight-gradient GEMM's
// the vocabulary.
#ifndef LP_DH_GROUP
#define LP_DH_GROUP 4
#endif
#ifndef LP_DW_GROUP
#define LP_DW_GROUP 4
#endif

template <class C, int G>
__global__ void __launch_bounds__(C::NT) k_dense_gemm_dtl(DenseGemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_ELEMS];
  const int per = g.n_mb * g.n_nb;
  const int ks = blockIdx.x / per;
  int mb, nb;
  tile_coords<G>(xcd_remap(blockIdx.x - ks * per, per), g.n_mb, g.n_nb, mb, nb);
  int rows = 0, K = g.K;
  if (g.count) {
    rows = tile_rows_of(g.count, g.tile_base, g.tile_rows, 0);
    if (g.k_from_count) {
      const int rows2 = g.ntiles > 1 ? tile_rows_of(g.count, g.tile_base, g.tile_rows, 1) : 0;
      K = rows2 > 0 ? static_cast<int>(g.tpad) + ((rows2 + 63) & ~63) : ((rows + 63) & ~63);
    }
  }
  const int M = g.m_from_count ? rows : g.M;
  const int m0 = mb * C::BM, n0 = nb * C::BN;
  if (m0 >= M) return;
  if (g.k_from_count && K == 0 && g.accumulate) return;
  const int kbeg = ks * g.ksplit;
  const int klen = (K - kbeg < g.ksplit) ? (K - kbeg) : g.ksplit;
  f32x16_t acc[C::MI][C::NI];
  const uint16_t* a = C::AKM ? g.a + m0 + static_cast<int64_t>(kbeg) * g.lda : g.a + static_cast<int64_t>(m0) * g.lda + kbeg;
  const uint16_t* b = C::BKM ? g.b + n0 + static_cast<int64_t>(kbeg) * g.ldb : g.b + static_cast<int64_t>(n0) * g.ldb + kbeg;
  gemm_tile_dtl_dense<C>(a, g.lda, M - m0, 0x7fffffff, b, g.ldb, g.N - n0, g.kvalid_b - kbeg, klen > 0 ? klen : 0, lds,
                         acc);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WGM, wn = wave / C::WGM;
  float* out = g.out + static_cast<int64_t>(ks) * g.tile_rows * g.ldo;  // splits > 1: partial ks
  const int mlane = m0 + wm * C::WTM + 4 * (lane >> 5);
  if (g.accumulate && m0 + C::BM <= M && n0 + C::BN <= g.N) {
    // full block, read-modify-write: all reads of a column group are issued
    // before any is consumed, so the block waits for memory once per group
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni) {
      float* col = out + (n0 + wn * C::WTN + ni * 32 + (lane & 31));
      float old[C::MI][16];
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          old[mi][i] = col[static_cast<int64_t>(mlane + mi * 32 + 8 * (i >> 2) + (i & 3)) * g.ldo];
#pragma unroll
      for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          col[static_cast<int64_t>(mlane + mi * 32 + 8 * (i >> 2) + (i & 3)) * g.ldo] = old[mi][i] + acc[mi][ni][i];
    }
    return;
  }
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int n = n0 + wn * C::WTN + ni * 32 + (lane & 31);
    if (n >= g.N) continue;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = mlane + mi * 32 + 8 * (i >> 2) + (i & 3);
        if (m < M) {
          float* p = out + static_cast<int64_t>(m) * g.ldo + n;
          *p = g.accumulate ? (*p + acc[mi][ni][i]) : acc[mi][ni][i];
        }
      }
  }
}

// Dense copy of a tile's hidden rows for the weight-gradient GEMM:
// dst[r][0, h) = src[idx[base + r]][0, h) for the tile's valid rows r, 0 for
// the other rows below nr_pad (h % 8 == 0, 16-byte aligned rows).
__global__ void __launch_bounds__(256) k_gather_rows_bf16(const uint16_t* __restrict__ src, int64_t ld,
                                                          const int* __restrict__ idx, const int* __restrict__ count,
                                                          int64_t base, int tile_rows, int nr_pad, int h,
                                                          uint16_t* __restrict__ dst) {
  const int rows = tile_rows_of(count, base, tile_rows, 0);
  const int nv = h / 8;
  for (int r = blockIdx.x; r < nr_pad; r += gridDim.x) {
    uint4* d = reinterpret_cast<uint4*>(dst + static_cast<int64_t>(r) * h);
    if (r < rows) {
      const uint4* sp = reinterpret_cast<const uint4*>(src + static_cast<int64_t>(idx[base + r]) * ld);
      for (int i = threadIdx.x; i < nv; i += 256) d[i] = sp[i];
    } else {
      for (int i = threadIdx.x; i < nv; i += 256) d[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

// dHidden[idx[base + m]][n] = sum over splits (in order) of partial[s][m][n].
__global__ void __launch_bounds__(256) k_splitk_reduce(const float* __restrict__ part, int splits, int tile_rows,
                                                       int h, const int* __restrict__ idx,
                                                       const int* __restrict__ count, int64_t tile_base,
                                                       float* __restrict__ out) {
  const int64_t rem = static_cast<int64_t>(*count) - tile_base;
  const int rows = static_cast<int>(rem < tile_rows ? (rem > 0 ? rem : 0) : tile_rows);
  const int64_t n = static_cast<int64_t>(rows) * h;
  const int64_t plane = static_cast<int64_t>(tile_rows) * h;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 4;
  for (int64_t e = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; e < n; e += stride) {
    // h % 8 == 0, so the 4 elements stay in one row
    float4 acc = *reinterpret_cast<const float4*>(part + e);
    for (int sp = 1; sp < splits; ++sp) {
      const float4 v = *reinterpret_cast<const float4*>(part + sp * plane + e);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const int64_t m = e / h;
    const int64_t col = e - m * h;
    *reinterpret_cast<float4*>(out + static_cast<int64_t>(idx[tile_base + m]) * h + col) = acc;
  }
}

// out rows: dst[row_of(m)][n] = D[m][n] (store) or += (accumulate).
struct OutGemmArgs {
  GemmOperands op;
  const int* count;    // device count (tile-relative rows) or nullptr
  int64_t tile_base;
  int tile_rows;
  int mode;            // 0: A rows = tile rows (M from count), K static; 1: K from count (rows8)
  const int* out_rows; // gather for output rows (indexes into idx) or nullptr
  float* out;
  int64_t ldo;
  int accumulate;
  int n_mb, n_nb;
};

template <class C>
__global__ void __launch_bounds__(C::NT) k_out_gemm(OutGemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  int mb, nb;
  tile_coords(xcd_remap(blockIdx.x, g.n_mb * g.n_nb), g.n_mb, g.n_nb, mb, nb);
  GemmOperands op = g.op;
  int rows = 0;
  if (g.count) {
    const int64_t rem = static_cast<int64_t>(*g.count) - g.tile_base;
    rows = static_cast<int>(rem < g.tile_rows ? (rem > 0 ? rem : 0) : g.tile_rows);
  }
  if (g.mode == 0) {
    op.M = rows;
  } else {
    op.K = (rows + 7) & ~7;
  }
  const int m0 = mb * C::BM, n0 = nb * C::BN;
  if (m0 >= op.M) return;
  if (g.mode == 1 && op.K == 0 && g.accumulate) return;
  GemmOperands opb = op;
  opb.a = op.a + static_cast<int64_t>(m0) * op.lda;
  opb.M = op.M - m0;
  if (op.b_rows == nullptr) {
    opb.b = op.b + static_cast<int64_t>(n0) * op.ldb;
  } else {
    opb.b_rows = op.b_rows + n0;
  }
  opb.N = op.N - n0;
  f32x16_t acc[C::MI][C::NI];
  gemm_tile<C>(opb, 0, 0, lds, acc);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WGM, wn = wave / C::WGM;
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int n = n0 + wn * C::WTN + ni * 32 + (lane & 31);
    if (n >= op.N) continue;
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + wm * C::WTM + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (m < op.M) {
          const int64_t orow = g.out_rows ? static_cast<int64_t>(g.out_rows[g.tile_base + m]) : static_cast<int64_t>(m);
          float* p = g.out + orow * g.ldo + n;
          *p = g.accumulate ? (*p + acc[mi][ni][i]) : acc[mi][ni][i];
        }
      }
  }
}

// First steps of both losses' backward: the scored-row list, and zeros in the
// hidden gradient of the unscored rows.
inline hipError_t backward_prologue(const LMHeadShape& sh, float* grad_hidden, int* idx, int* count, hipStream_t s) {
  {
    TimedLaunch tl("k_compact", s);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, s, sh.mask, sh.T, idx, count, zero_outs());
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !grad_hidden) return e;
  {
    TimedLaunch tl("k_zero_unscored_rows", s);
    const unsigned blocks = static_cast<unsigned>(sh.T < 65536 ? sh.T : 65536);
    hipLaunchKernelGGL(k_zero_unscored_rows, dim3(blocks), dim3(256), 0, s, sh.mask, sh.T, sh.h, grad_hidden);
  }
  return hipGetLastError();
}

// Generic tiles (any h % 8 == 0): per tile of rows, dL/dlogits (launched by
// `launch_dz`) in both [row][vocab] and [vocab][row] order, then dHidden and
// dW as NT GEMMs against a once-per-call W^T and the tile's H^T.
template <class LaunchDz>
hipError_t backward_tiles_generic(const LMHeadShape& sh, float* grad_hidden, float* grad_weight, char* ws,
                                  const LMHeadWorkspace& w, hipStream_t s, LaunchDz&& launch_dz) {
  using C = BwdCfg;
  int* idx = reinterpret_cast<int*>(ws + w.idx_off);
  int* count = reinterpret_cast<int*>(ws + w.count_off);
  const int64_t tr = sh.tile_rows < sh.T ? sh.tile_rows : sh.T;
  const int64_t tpad = static_cast<int64_t>(align_up(static_cast<size_t>(tr), 64));
  const int64_t vpad = w.vpad;
  const BwdBuffers bb = bwd_buffers(ws + w.dz_off, tr, sh.h, vpad);
  hipError_t e = backward_prologue(sh, grad_hidden, idx, count, s);
  if (e != hipSuccess) return e;
  if (grad_hidden) {
    // W^T [h x vpad], zero past V
    dim3 g(static_cast<unsigned>((vpad + 63) / 64), static_cast<unsigned>((sh.h + 63) / 64));
    {
      TimedLaunch tl("k_transpose_bf16", s);
      hipLaunchKernelGGL(k_transpose_bf16, g, dim3(256), 0, s, sh.weight, sh.ld_w, static_cast<const int*>(nullptr),
                         static_cast<const int*>(nullptr), int64_t(0), sh.V, sh.V, static_cast<int>(vpad), sh.h, bb.wt,
                         vpad);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int n_vb = (sh.V + C::BM - 1) / C::BM;
  const int n_nb = static_cast<int>((tr + C::BN - 1) / C::BN);
  for (int64_t base = 0; base < sh.T; base += tr) {
    if ((e = launch_dz(base, tr, tpad, vpad, n_vb, n_nb, idx, count, bb.dz, grad_weight ? bb.dzt : nullptr)) !=
        hipSuccess)
      return e;
    if (grad_hidden) {
      // dHidden[idx[r]] = dZ[r] . W  :  A = dZ [rows x vpad], B = W^T [h x vpad], K = vpad
      OutGemmArgs g;
      g.op.a = bb.dz;
      g.op.lda = vpad;
      g.op.M = 0;
      g.op.b = bb.wt;
      g.op.ldb = vpad;
      g.op.b_rows = nullptr;
      g.op.N = sh.h;
      g.op.K = static_cast<int>(vpad);
      g.count = count;
      g.tile_base = base;
      g.tile_rows = static_cast<int>(tr);
      g.mode = 0;
      g.out_rows = idx;
      g.out = grad_hidden;
      g.ldo = sh.h;
      g.accumulate = 0;
      g.n_mb = static_cast<int>((tr + C::BM - 1) / C::BM);
      g.n_nb = (sh.h + C::BN - 1) / C::BN;
      {
        TimedLaunch tl("k_out_gemm_dhidden", s);
        hipLaunchKernelGGL(k_out_gemm<C>, dim3(static_cast<unsigned>(g.n_mb) * g.n_nb), dim3(C::NT), 0, s, g);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (grad_weight) {
      // H_tile^T [h x tpad], zero past the tile's rows
      dim3 gt(static_cast<unsigned>(tpad / 64), static_cast<unsigned>((sh.h + 63) / 64));
      {
        TimedLaunch tl("k_transpose_bf16", s);
        hipLaunchKernelGGL(k_transpose_bf16, gt, dim3(256), 0, s, sh.hidden, sh.ld_h, static_cast<const int*>(idx),
                           static_cast<const int*>(count), base, 0, static_cast<int>(tr), static_cast<int>(tpad), sh.h,
                           bb.ht, tpad);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      // dW (+)= dZ^T . H_tile : A = dZ^T [V x tpad], B = H_tile^T [h x tpad], K = rows8
      OutGemmArgs g;
      g.op.a = bb.dzt;
      g.op.lda = tpad;
      g.op.M = sh.V;
      g.op.b = bb.ht;
      g.op.ldb = tpad;
      g.op.b_rows = nullptr;
      g.op.N = sh.h;
      g.op.K = 0;
      g.count = count;
      g.tile_base = base;
      g.tile_rows = static_cast<int>(tr);
      g.mode = 1;
      g.out_rows = nullptr;
      g.out = grad_weight;
      g.ldo = sh.h;
      g.accumulate = base == 0 ? 0 : 1;
      g.n_mb = (sh.V + C::BM - 1) / C::BM;
      g.n_nb = (sh.h + C::BN - 1) / C::BN;
      {
        TimedLaunch tl("k_out_gemm_dweight", s);
        hipLaunchKernelGGL(k_out_gemm<C>, dim3(static_cast<unsigned>(g.n_mb) * g.n_nb), dim3(C::NT), 0, s, g);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Direct-to-LDS tiles (h % 64 == 0 and 32-bit offsets): per tile of rows,
// dL/dlogits [row][vocab] only (launched by `launch_dz`, rows zero-padded up
// to a multiple of 64), the tile's hidden rows copied densely, dHidden = dZ .
// W on W as stored, and dW = dZ^T . H once per pair of consecutive tiles
// (each tile's dZ and hidden rows go to one half of a two-tile buffer), so
// the fp32 dW is read and written half as often.  No transposed copy of any
// operand is made.
template <class LaunchDz>
hipError_t backward_tiles_fast(const LMHeadShape& sh, int bm, int bn, float* grad_hidden, float* grad_weight,
                               char* ws, const LMHeadWorkspace& w, hipStream_t s, LaunchDz&& launch_dz) {
  using FH = DenseDhCfg;
  using FW = DenseDwCfg;
  int* idx = reinterpret_cast<int*>(ws + w.idx_off);
  int* count = reinterpret_cast<int*>(ws + w.count_off);
  const int64_t tr = sh.tile_rows < sh.T ? sh.tile_rows : sh.T;
  const int64_t tpad = static_cast<int64_t>(align_up(static_cast<size_t>(tr), 64));
  const int64_t vpad = w.vpad;
  const BwdBuffers bb = bwd_buffers(ws + w.dz_off, tr, sh.h, vpad);
  // two tiles per dW launch when K of both still fits the 32-bit offsets
  const int pair = dense_fast(vpad, tpad, sh.h, sh.ld_w, 2) ? 2 : 1;
  hipError_t e = backward_prologue(sh, grad_hidden, idx, count, s);
  if (e != hipSuccess) return e;
  const int n_vb = (sh.V + bm - 1) / bm;
  const int n_nb = static_cast<int>((tr + bn - 1) / bn);
  int t = 0;
  for (int64_t base = 0; base < sh.T; base += tr, ++t) {
    const int slot = t % pair;
    uint16_t* dz = bb.dz2 + slot * tpad * vpad;
    if ((e = launch_dz(base, tr, tpad, vpad, n_vb, n_nb, idx, count, dz, nullptr)) != hipSuccess) return e;
    if (grad_hidden) {
      // dHidden[idx[r]] = dZ[r] . W : K = vpad split into kSplitK ranges, then a fixed-order sum
      DenseGemmArgs g;
      g.a = dz;
      g.lda = vpad;
      g.M = 0;
      g.b = sh.weight;
      g.ldb = sh.ld_w;
      g.N = sh.h;
      g.K = static_cast<int>(vpad);
      g.kvalid_b = sh.V;
      g.count = count;
      g.tile_base = base;
      g.tile_rows = static_cast<int>(tr);
      g.tpad = tpad;
      g.ntiles = 1;
      g.m_from_count = 1;
      g.k_from_count = 0;
      g.splits = kSplitK;
      g.ksplit = static_cast<int>(align_up(static_cast<size_t>((vpad + kSplitK - 1) / kSplitK), 64));
      g.out = bb.hpart;
      g.ldo = sh.h;
      g.accumulate = 0;
      g.n_mb = static_cast<int>((tr + FH::BM - 1) / FH::BM);
      g.n_nb = (sh.h + FH::BN - 1) / FH::BN;
      {
        TimedLaunch tl("k_out_gemm_dhidden", s);
        hipLaunchKernelGGL((k_dense_gemm_dtl<FH, LP_DH_GROUP>), dim3(static_cast<unsigned>(g.n_mb) * g.n_nb * kSplitK),
                           dim3(FH::NT), 0, s, g);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      {
        TimedLaunch tl("k_splitk_reduce", s);
        const int64_t n4 = tr * sh.h / 4;
        const unsigned blocks = static_cast<unsigned>(n4 < 65536 * 256 ? (n4 + 255) / 256 : 65536);
        hipLaunchKernelGGL(k_splitk_reduce, dim3(blocks), dim3(256), 0, s, bb.hpart, kSplitK, static_cast<int>(tr),
                           sh.h, static_cast<const int*>(idx), static_cast<const int*>(count), base, grad_hidden);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (grad_weight) {
      {
        TimedLaunch tl("k_gather_rows", s);
        const unsigned blocks = static_cast<unsigned>(tpad < 65536 ? tpad : 65536);
        hipLaunchKernelGGL(k_gather_rows_bf16, dim3(blocks), dim3(256), 0, s, sh.hidden, sh.ld_h,
                           static_cast<const int*>(idx), static_cast<const int*>(count), base, static_cast<int>(tr),
                           static_cast<int>(tpad), sh.h, bb.ht2 + slot * tpad * sh.h);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (slot == pair - 1 || base + tr >= sh.T) {
        // dW (+)= dZ^T . H over the rows of this launch's tiles
        const int64_t base0 = base - slot * tr;
        DenseGemmArgs g;
        g.a = bb.dz2;
        g.lda = vpad;
        g.M = sh.V;
        g.b = bb.ht2;
        g.ldb = sh.h;
        g.N = sh.h;
        g.K = 0;
        g.kvalid_b = 0x7fffffff;
        g.count = count;
        g.tile_base = base0;
        g.tile_rows = static_cast<int>(tr);
        g.tpad = tpad;
        g.ntiles = slot + 1;
        g.m_from_count = 0;
        g.k_from_count = 1;
        g.splits = 1;
        g.ksplit = static_cast<int>(pair * tpad);
        g.out = grad_weight;
        g.ldo = sh.h;
        g.accumulate = base0 == 0 ? 0 : 1;
        g.n_mb = (sh.V + FW::BM - 1) / FW::BM;
        g.n_nb = (sh.h + FW::BN - 1) / FW::BN;
        {
          TimedLaunch tl("k_out_gemm_dweight", s);
          hipLaunchKernelGGL((k_dense_gemm_dtl<FW, LP_DW_GROUP>), dim3(static_cast<unsigned>(g.n_mb) * g.n_nb), dim3(FW::NT), 0, s,
                             g);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
  }
  return hipSuccess;
}

template <class LaunchDz>
hipError_t backward_tiles(const LMHeadShape& sh, bool fast, int bm_fast, int bn_fast, float* grad_hidden,
                          float* grad_weight, char* ws, const LMHeadWorkspace& w, hipStream_t s,
                          LaunchDz&& launch_dz) {
  if (fast) return backward_tiles_fast(sh, bm_fast, bn_fast, grad_hidden, grad_weight, ws, w, s, launch_dz);
  return backward_tiles_generic(sh, grad_hidden, grad_weight, ws, w, s, launch_dz);
}


hipError_t launch_lmhead_backward(const LMHeadShape& sh, const float* lse, const float* entropy,
                                  const float* grad_logprob, const float* grad_entropy, float* grad_hidden,
                                  float* grad_weight, char* ws, const LMHeadWorkspace& w, hipStream_t s) {
  const bool fast = lmhead_fast_tiles(sh.T, sh.h, sh.V, sh.ld_h, sh.ld_w, sh.tile_rows, 1) &&
                    (reinterpret_cast<uintptr_t>(grad_hidden) & 15u) == 0;
  auto launch_dz = [&](int64_t base, int64_t tr, int64_t tpad, int64_t vpad, int n_vb, int n_nb, const int* idx,
                       const int* count, uint16_t* dz, uint16_t* dzt) -> hipError_t {
    DzArgs d;
    d.weight = sh.weight;
    d.ld_w = sh.ld_w;
    d.hidden = sh.hidden;
    d.ld_h = sh.ld_h;
    d.h = sh.h;
    d.V = sh.V;
    d.vpad = vpad;
    d.idx = idx;
    d.count = count;
    d.targets = sh.targets;
    d.K = sh.K;
    d.lse = lse;
    d.entropy = entropy;
    d.g_lp = grad_logprob;
    d.g_H = grad_entropy;
    d.c = sh.c;
    d.inv_tau = sh.inv_tau;
    d.tile_base = base;
    d.tile_rows = static_cast<int>(tr);
    d.tpad = tpad;
    d.n_vb = n_vb;
    d.n_nb = n_nb;
    d.dz = dz;
    d.dzt = dzt;
    TimedLaunch tl("k_bwd_dz", s);
    const dim3 grid(static_cast<unsigned>(n_vb) * n_nb);
    if (fast)
      hipLaunchKernelGGL(k_bwd_dz_dtl<BwdDtlCfg>, grid, dim3(BwdDtlCfg::NT), 0, s, d);
    else
      hipLaunchKernelGGL(k_bwd_dz<BwdCfg>, grid, dim3(BwdCfg::NT), 0, s, d);
    return hipGetLastError();
  };
  return backward_tiles(sh, fast, BwdDtlCfg::BM, BwdDtlCfg::BN, grad_hidden, grad_weight, ws, w, s, launch_dz);
}


// ---------------------------------------------------------------------------
// KL(teacher || student) with both logits rebuilt through each model's head
// ---------------------------------------------------------------------------
// DeepSeek-V4 book ch.19 (名词速通 "不实例化 logits", §2 "Teacher
// Scheduling"): only the last hidden states are kept; the logits of both
// models are rebuilt through their output heads a tile at a time and reduced
// to the exact KL directly.  Fast path, per chunk of scored rows: a teacher
// pass (GEMM v, stored as fp32 in accumulator order) and a student pass
// (GEMM u, whose epilogue reads v back and folds both into one dual state per
// (row, vocab block), the state of the KL on given logits); a merge kernel
// combines a row's states in a fixed order.  The generic tile runs both GEMMs
// into two accumulator sets in one kernel.  The backward recomputes both and
// writes dL/du = g (p_u - p_v) as bf16 for the student's dHidden / dW GEMMs;
// the teacher is not trained.

// Vocab blocks per group in the KL tiles' walk.
#ifndef LP_KL_GROUP_V
#define LP_KL_GROUP_V 4
#endif
constexpr int kKLGroupV = LP_KL_GROUP_V;
static_assert(KLCfg::BM >= (FwdCfg::BM < FwdDtlCfg::BM ? FwdCfg::BM : FwdDtlCfg::BM),
              "the workspace holds partial states for vocab blocks of at least the smallest forward block");

struct KLHeadArgs {
  const uint16_t* ws;  // student weight [V x ld_ws]
  int64_t ld_ws;
  const uint16_t* hs;  // student hidden [T x ld_hs]
  int64_t ld_hs;
  int h_s;
  const uint16_t* wt;  // teacher weight
  int64_t ld_wt;
  const uint16_t* ht;  // teacher hidden
  int64_t ld_ht;
  int h_t;
  int V;
  const int* idx;
  const int* count;
  const int64_t* targets;  // [T] or nullptr
  float c;                 // log2 e
  int64_t tile_base;
  int tile_rows;
  int n_vb, n_nb;
  float* part;  // [tile_rows][n_vb][5]
  float* zy;    // [tile_rows][2]: student, teacher target logit
  float* tbuf;  // teacher logits of the chunk (two-pass tiles)
};

// Where the student epilogues find the teacher's logits of their block: in
// registers (both GEMMs in one kernel), or in the chunk buffer the teacher
// pass wrote in accumulator order.  column(ni, x) yields x[mi][i] =
// teacher logit at accumulator (mi, ni, i) of this lane.
template <class C>
struct TeacherRegs {
  f32x16_t (&acc)[C::MI][C::NI];
  __device__ __forceinline__ void column(int ni, float (&x)[C::MI][16]) {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[mi][i] = acc[mi][ni][i];
  }
};

// Accumulator-order buffer of one BM x BN block: wave w's sub-tile at
// w * WTM * WTN floats, inside it [mi][ni][quad][lane][4], so each 16-byte
// store or load of a wave covers 1 KB contiguously.
template <class C>
__device__ __forceinline__ int64_t tbuf_block(int vb, int nb, int n_nb) {
  return (static_cast<int64_t>(vb) * n_nb + nb) * (C::BM * C::BN);
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
// The chunk buffer is written once and read once, far apart: non-temporal
// accesses keep it from evicting the weight and hidden strips the tiles share
// in L2 (measured 2 % faster).
#ifndef LP_KL_TBUF_NT
#define LP_KL_TBUF_NT 1
#endif

template <class C>
__device__ __forceinline__ void tbuf_store(float* blk, const f32x16_t (&acc)[C::MI][C::NI]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* p = blk + wave * (C::WTM * C::WTN) + 4 * lane;
#pragma unroll
  for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t v{acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2], acc[mi][ni][4 * q + 3]};
        f32x4_t* d = reinterpret_cast<f32x4_t*>(p + ((mi * C::NI + ni) * 4 + q) * 256);
        if (LP_KL_TBUF_NT)
          __builtin_nontemporal_store(v, d);
        else
          *d = v;
      }
}

// Column ni + 1 is loaded while column ni is folded.
template <class C>
struct TeacherMem {
  const float* p;  // block base + this wave's sub-tile + 4 * lane
  f32x4_t nxt[C::MI][4];
  __device__ __forceinline__ TeacherMem(const float* blk) {
    p = blk + (threadIdx.x >> 6) * (C::WTM * C::WTN) + 4 * (threadIdx.x & 63);
    load(0);
  }
  __device__ __forceinline__ void load(int ni) {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p + ((mi * C::NI + ni) * 4 + q) * 256);
        nxt[mi][q] = LP_KL_TBUF_NT ? __builtin_nontemporal_load(src) : *src;
      }
  }
  __device__ __forceinline__ void column(int ni, float (&x)[C::MI][16]) {
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[mi][4 * q] = nxt[mi][q][0];
        x[mi][4 * q + 1] = nxt[mi][q][1];
        x[mi][4 * q + 2] = nxt[mi][q][2];
        x[mi][4 * q + 3] = nxt[mi][q][3];
      }
    if (ni + 1 < C::NI) load(ni + 1);
  }
};

template <class C, class TSrc>
__device__ __forceinline__ void kl_epilogue(const KLHeadArgs& a, f32x16_t (&accu)[C::MI][C::NI], TSrc& tv, int vb,
                                            int n0, int rows, uint16_t* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WGM, wn = wave / C::WGM;
  const int vwave = vb * C::BM + wm * C::WTM;
  const int half = lane >> 5;
  KLState* sm = reinterpret_cast<KLState*>(lds);  // [WGM][BN], reused after the K loops
  const float c = a.c;
  const bool full_block = (vb + 1) * C::BM <= a.V;
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int nl = wn * C::WTN + ni * 32 + (lane & 31);
    const int r = n0 + nl;
    const bool valid_row = r < rows;
    KLState st{kNegBig, 0.f, kNegBig, 0.f, 0.f};
    float tcol[C::MI][16];
    tv.column(ni, tcol);
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi) {
      float xu[16], xv[16];
      if (full_block) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          xu[i] = accu[mi][ni][i];
          xv[i] = tcol[mi][i];
        }
        kl_push<false, 16, 16>(st, xu, xv, c);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = vwave + mi * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          xu[i] = (v < a.V) ? accu[mi][ni][i] : -INFINITY;
          xv[i] = (v < a.V) ? tcol[mi][i] : -INFINITY;
        }
        kl_push<true, 16, 16>(st, xu, xv, c);
      }
    }
    if (a.targets && valid_row) {
      const int64_t yrel = a.targets[a.idx[a.tile_base + r]] - vwave;
      if (yrel >= 0 && yrel < C::WTM) {
        float zu = 0.f, zv = 0.f;
        bool found = false;
#pragma unroll
        for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (yrel == mi * 32 + 8 * (i >> 2) + 4 * half + (i & 3)) {
              zu = accu[mi][ni][i];
              zv = tcol[mi][i];
              found = true;
            }
        if (found) {
          a.zy[static_cast<int64_t>(r) * 2] = zu;
          a.zy[static_cast<int64_t>(r) * 2 + 1] = zv;
        }
      }
    }
    KLState o;
    o.mcu = __shfl_xor(st.mcu, 32, 64);
    o.su = __shfl_xor(st.su, 32, 64);
    o.mcv = __shfl_xor(st.mcv, 32, 64);
    o.sv = __shfl_xor(st.sv, 32, 64);
    o.C = __shfl_xor(st.C, 32, 64);
    st = kl_merge(st, o);
    if (lane < 32) sm[wm * C::BN + nl] = st;
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int ni = 0; ni < C::NI; ++ni) {
      const int nl = wn * C::WTN + ni * 32 + lane;
      const int r = n0 + nl;
      if (r < rows) {
        KLState st = sm[nl];
#pragma unroll
        for (int k = 1; k < C::WGM; ++k) st = kl_merge(st, sm[k * C::BN + nl]);
        float* p = a.part + (static_cast<int64_t>(r) * a.n_vb + vb) * 5;
        p[0] = st.mcu;
        p[1] = st.su;
        p[2] = st.mcv;
        p[3] = st.sv;
        p[4] = st.C;
      }
    }
  }
}

// Block coordinates shared by the KL tiles; false if the block has no rows.
__device__ __forceinline__ bool kl_block(int n_vb, int n_nb, const int* count_p, int64_t tile_base, int tile_rows,
                                         int bn, int& vb, int& n0, int& rows) {
  int nb;
  tile_coords<kKLGroupV>(xcd_remap(blockIdx.x, n_vb * n_nb), n_vb, n_nb, vb, nb);
  const int64_t rem = static_cast<int64_t>(*count_p) - tile_base;
  rows = static_cast<int>(rem < tile_rows ? rem : tile_rows);
  n0 = nb * bn;
  return n0 < rows;
}

// Generic KL tile (any h % 8 == 0).
template <class C>
__global__ void __launch_bounds__(C::NT) k_kl_tile(KLHeadArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  int vb, n0, rows;
  if (!kl_block(a.n_vb, a.n_nb, a.count, a.tile_base, a.tile_rows, C::BN, vb, n0, rows)) return;
  const int v0 = vb * C::BM;
  GemmOperands op;
  op.a = a.wt + static_cast<int64_t>(v0) * a.ld_wt;
  op.lda = a.ld_wt;
  op.M = a.V - v0;
  op.b = a.ht;
  op.ldb = a.ld_ht;
  op.b_rows = a.idx + a.tile_base + n0;
  op.N = rows - n0;
  op.K = a.h_t;
  f32x16_t accv[C::MI][C::NI], accu[C::MI][C::NI];
  gemm_tile<C>(op, 0, 0, lds, accv);
  op.a = a.ws + static_cast<int64_t>(v0) * a.ld_ws;
  op.lda = a.ld_ws;
  op.b = a.hs;
  op.ldb = a.ld_hs;
  op.K = a.h_s;
  gemm_tile<C>(op, 0, 0, lds, accu);
  TeacherRegs<C> tv{accv};
  kl_epilogue<C>(a, accu, tv, vb, n0, rows, lds);
}

// Fast path, pass 1 (both h % 64 == 0): the teacher's logits of the chunk,
// stored in accumulator order.
template <class C>
__global__ void __launch_bounds__(C::NT) k_kl_teacher_dtl(KLHeadArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_ELEMS];
  int vb, n0, rows;
  if (!kl_block(a.n_vb, a.n_nb, a.count, a.tile_base, a.tile_rows, C::BN, vb, n0, rows)) return;
  const int v0 = vb * C::BM;
  f32x16_t acc[C::MI][C::NI];
  gemm_tile_dtl<C>(a.wt + static_cast<int64_t>(v0) * a.ld_wt, a.ld_wt, a.V - v0, a.ht, a.ld_ht,
                   a.idx + a.tile_base + n0, rows - n0, a.h_t, lds, acc);
  tbuf_store<C>(a.tbuf + tbuf_block<C>(vb, n0 / C::BN, a.n_nb), acc);
}

// Fast path, pass 2: the student's logits, folded with the stored teacher
// logits into one dual state per (row, vocab block).
template <class C>
__global__ void __launch_bounds__(C::NT) k_kl_student_dtl(KLHeadArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::LDS_ELEMS];
  int vb, n0, rows;
  if (!kl_block(a.n_vb, a.n_nb, a.count, a.tile_base, a.tile_rows, C::BN, vb, n0, rows)) return;
  const int v0 = vb * C::BM;
  f32x16_t accu[C::MI][C::NI];
  gemm_tile_dtl<C>(a.ws + static_cast<int64_t>(v0) * a.ld_ws, a.ld_ws, a.V - v0, a.hs, a.ld_hs,
                   a.idx + a.tile_base + n0, rows - n0, a.h_s, lds, accu);
  TeacherMem<C> tv(a.tbuf + tbuf_block<C>(vb, n0 / C::BN, a.n_nb));
  kl_epilogue<C>(a, accu, tv, vb, n0, rows, lds);
}

struct KLMergeArgs {
  const float* part;
  const float* zy;
  int n_vb;
  const int* idx;
  const int* count;
  const int64_t* targets;
  const uint8_t* diff_mask;
  int V;
  float c;
  int64_t tile_base;
  int tile_rows;
  KLHeadOutputs out;
};

__global__ void __launch_bounds__(256) k_kl_merge(KLMergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rem = static_cast<int64_t>(*a.count) - a.tile_base;
  const int rows = static_cast<int>(rem < a.tile_rows ? rem : a.tile_rows);
  if (r >= rows) return;
  const float* p = a.part + static_cast<int64_t>(r) * a.n_vb * 5;
  KLState st{kNegBig, 0.f, kNegBig, 0.f, 0.f};
  for (int vb = lane; vb < a.n_vb; vb += 64)
    st = kl_merge(st, KLState{p[vb * 5], p[vb * 5 + 1], p[vb * 5 + 2], p[vb * 5 + 3], p[vb * 5 + 4]});
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
  if (lane != 0) return;
  const int64_t row = a.idx[a.tile_base + r];
  const float l2u = log2f(st.su), l2v = log2f(st.sv);
  const float lseu = (st.mcu + l2u) * kLn2, lsev = (st.mcv + l2v) * kLn2;
  const KLHeadOutputs& o = a.out;
  o.kl[row] = st.C / st.sv - ((st.mcv - st.mcu) + (l2v - l2u)) * kLn2;
  if (o.lse_student) o.lse_student[row] = lseu;
  if (o.lse_teacher) o.lse_teacher[row] = lsev;
  if (a.targets) {
    const int64_t y = a.targets[row];
    float lpu = __builtin_nanf(""), lpv = __builtin_nanf("");
    if (y >= 0 && y < a.V) {
      lpu = (fmaf(a.zy[static_cast<int64_t>(r) * 2], a.c, -st.mcu) - l2u) * kLn2;
      lpv = (fmaf(a.zy[static_cast<int64_t>(r) * 2 + 1], a.c, -st.mcv) - l2v) * kLn2;
    }
    if (o.lp_student) o.lp_student[row] = lpu;
    if (o.lp_teacher) o.lp_teacher[row] = lpv;
    if (o.prob_diff) {
      const bool keep = a.diff_mask == nullptr || a.diff_mask[row] != 0;
      o.prob_diff[row] = keep ? fabsf(expf(lpu) - expf(lpv)) : 0.f;
    }
  }
}

// Both heads on the direct-to-LDS tiles; the backward's dense GEMMs run on
// the student's dZ buffers.
static bool kl_fast_path(const LMHeadShape& st, const LMHeadShape& te, int backward) {
  return lmhead_fast_tiles(st.T, st.h, st.V, st.ld_h, st.ld_w, st.tile_rows, backward) &&
         lmhead_fast_path(te);
}

static KLHeadArgs kl_args(const LMHeadShape& st, const LMHeadShape& te) {
  KLHeadArgs a;
  a.ws = st.weight;
  a.ld_ws = st.ld_w;
  a.hs = st.hidden;
  a.ld_hs = st.ld_h;
  a.h_s = st.h;
  a.wt = te.weight;
  a.ld_wt = te.ld_w;
  a.ht = te.hidden;
  a.ld_ht = te.ld_h;
  a.h_t = te.h;
  a.V = st.V;
  a.c = 1.44269504088896340736f;
  return a;
}

hipError_t launch_lmhead_kl_forward(const LMHeadShape& sh, const LMHeadShape& te, const int64_t* targets,
                                    const uint8_t* diff_mask, const KLHeadOutputs& out, char* ws,
                                    const LMHeadWorkspace& w, hipStream_t s) {
  int* idx = reinterpret_cast<int*>(ws + w.idx_off);
  int* count = reinterpret_cast<int*>(ws + w.count_off);
  float* part = reinterpret_cast<float*>(ws + w.part_off);
  float* zy = reinterpret_cast<float*>(ws + w.zy_off);
  {
    TimedLaunch tl("k_compact", s);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, s, sh.mask, sh.T, idx, count,
                       zero_outs(out.kl, 1, out.lp_student, out.lp_teacher, out.prob_diff, out.lse_student,
                                 out.lse_teacher));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool fast = kl_fast_path(sh, te, 0);
  // chunks of at most kKLChunk rows (the fast path's teacher buffer holds one)
  const int64_t tr0 = sh.tile_rows < sh.T ? sh.tile_rows : sh.T;
  const int64_t tr = tr0 > kKLChunk ? kKLChunk : tr0;
  const int bm = fast ? KLCfg::BM : FwdCfg::BM;
  const int bn = fast ? KLCfg::BN : FwdCfg::BN;
  const int n_vb = (sh.V + bm - 1) / bm;
  const int n_nb = static_cast<int>((tr + bn - 1) / bn);
  for (int64_t base = 0; base < sh.T; base += tr) {
    KLHeadArgs a = kl_args(sh, te);
    a.idx = idx;
    a.count = count;
    a.targets = targets;
    a.tile_base = base;
    a.tile_rows = static_cast<int>(tr);
    a.n_vb = n_vb;
    a.n_nb = n_nb;
    a.part = part;
    a.zy = zy;
    a.tbuf = reinterpret_cast<float*>(ws + w.tbuf_off);
    const dim3 grid(static_cast<unsigned>(n_vb) * n_nb);
    if (fast) {
      {
        TimedLaunch tl("k_kl_teacher", s);
        hipLaunchKernelGGL(k_kl_teacher_dtl<KLCfg>, grid, dim3(KLCfg::NT), 0, s, a);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      TimedLaunch tl("k_kl_student", s);
      hipLaunchKernelGGL(k_kl_student_dtl<KLCfg>, grid, dim3(KLCfg::NT), 0, s, a);
    } else {
      TimedLaunch tl("k_kl_tile", s);
      hipLaunchKernelGGL(k_kl_tile<FwdCfg>, grid, dim3(FwdCfg::NT), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    KLMergeArgs m;
    m.part = part;
    m.zy = zy;
    m.n_vb = n_vb;
    m.idx = idx;
    m.count = count;
    m.targets = targets;
    m.diff_mask = diff_mask;
    m.V = sh.V;
    m.c = a.c;
    m.tile_base = base;
    m.tile_rows = static_cast<int>(tr);
    m.out = out;
    {
      TimedLaunch tl("k_kl_merge", s);
      hipLaunchKernelGGL(k_kl_merge, dim3(static_cast<unsigned>((tr + 3) / 4)), dim3(256), 0, s, m);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---- KL backward: dL/du = g (p_u - p_v) on the student's logits -----------

struct KLDzArgs {
  KLHeadArgs h;
  int64_t vpad;
  const float* lse_u;
  const float* lse_v;
  const float* g;
  int64_t tpad;
  uint16_t* dz;
  uint16_t* dzt;
};

template <class C, bool STAGED, class TSrc>
__device__ __forceinline__ void kl_dz_epilogue(const KLDzArgs& a, f32x16_t (&accu)[C::MI][C::NI], TSrc& tv, int v0,
                                               int n0, int rows, int rowsK, uint16_t* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave % C::WGM, wn = wave / C::WGM;
  const int vlane = v0 + wm * C::WTM + 4 * (lane >> 5);
  const float c = a.h.c;
#pragma unroll
  for (int ni = 0; ni < C::NI; ++ni) {
    const int r = n0 + wn * C::WTN + ni * 32 + (lane & 31);
    float tcol[C::MI][16];
    tv.column(ni, tcol);  // before the row test: keeps the column prefetch uniform
    if (r >= rowsK) continue;
    const bool valid = r < rows;
    float lu = 0.f, lv = 0.f, g = 0.f;
    if (valid) {
      const int64_t row = a.h.idx[a.h.tile_base + r];
      lu = a.lse_u[row] * c;
      lv = a.lse_v[row] * c;
      g = a.g[row];
    }
#pragma unroll
    for (int mi = 0; mi < C::MI; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int vq = vlane + mi * 32 + 8 * q;
        float dv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float d = 0.f;
          if (valid && vq + j < a.h.V) {
            const float pu = fast_exp2(fmaf(accu[mi][ni][q * 4 + j], c, -lu));
            const float pv = fast_exp2(fmaf(tcol[mi][q * 4 + j], c, -lv));
            d = g * (pu - pv);
          }
          dv[j] = d;
        }
        const uint2 pk = pack_bf16x4(dv);
        if (STAGED)
          dz_stage4(lds, DzStage<C>::P, r - n0, vq - v0, pk);
        else if (vq < a.vpad)
          dz_store4(a.dz, a.dzt, a.vpad, a.tpad, r, vq, pk);
      }
  }
  if (STAGED) {
    __syncthreads();
    const int nrow = (rowsK - n0) < C::BN ? (rowsK - n0) : C::BN;
    dz_flush_rows<C>(lds, a.dz, a.vpad, v0, n0, nrow);
    if (a.dzt) dzt_flush_cols<C>(lds, a.dzt, a.tpad, a.vpad, v0, n0, nrow);
  }
}

template <class C>
__global__ void __launch_bounds__(C::NT) k_kl_dz(KLDzArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  int vb, n0, rows;
  kl_block(a.h.n_vb, a.h.n_nb, a.h.count, a.h.tile_base, a.h.tile_rows, C::BN, vb, n0, rows);
  const int rowsK = (rows + 7) & ~7;
  if (rows <= 0 || n0 >= rowsK) return;
  const int v0 = vb * C::BM;
  GemmOperands op;
  op.a = a.h.wt + static_cast<int64_t>(v0) * a.h.ld_wt;
  op.lda = a.h.ld_wt;
  op.M = a.h.V - v0;
  op.b = a.h.ht;
  op.ldb = a.h.ld_ht;
  op.b_rows = a.h.idx + a.h.tile_base + n0;
  op.N = rows - n0;
  op.K = a.h.h_t;
  f32x16_t accv[C::MI][C::NI], accu[C::MI][C::NI];
  gemm_tile<C>(op, 0, 0, lds, accv);
  op.a = a.h.ws + static_cast<int64_t>(v0) * a.h.ld_ws;
  op.lda = a.h.ld_ws;
  op.b = a.h.hs;
  op.ldb = a.h.ld_hs;
  op.K = a.h.h_s;
  gemm_tile<C>(op, 0, 0, lds, accu);
  TeacherRegs<C> tv{accv};
  kl_dz_epilogue<C, false>(a, accu, tv, v0, n0, rows, rowsK, lds);
}

// Fast path, pass 2 of the backward (pass 1 is k_kl_teacher_dtl): the
// student's logits against the stored teacher logits; the chunk's rows are
// zero-padded up to a multiple of 64.
template <class C>
__global__ void __launch_bounds__(C::NT) k_kl_dz_student_dtl(KLDzArgs a) {
  constexpr int kLds = C::LDS_ELEMS > DzStage<C>::ELEMS ? C::LDS_ELEMS : DzStage<C>::ELEMS;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kLds];
  int vb, n0, rows;
  kl_block(a.h.n_vb, a.h.n_nb, a.h.count, a.h.tile_base, a.h.tile_rows, C::BN, vb, n0, rows);
  const int rowsK = (rows + 63) & ~63;
  if (rows <= 0 || n0 >= rowsK) return;  // n0 < rowsK implies n0 < rows: the teacher pass ran this block
  const int v0 = vb * C::BM;
  f32x16_t accu[C::MI][C::NI];
  gemm_tile_dtl<C>(a.h.ws + static_cast<int64_t>(v0) * a.h.ld_ws, a.h.ld_ws, a.h.V - v0, a.h.hs, a.h.ld_hs,
                   a.h.idx + a.h.tile_base + n0, rows - n0, a.h.h_s, lds, accu);
  TeacherMem<C> tv(a.h.tbuf + tbuf_block<C>(vb, n0 / C::BN, a.h.n_nb));
  kl_dz_epilogue<C, true>(a, accu, tv, v0, n0, rows, rowsK, lds);
}

hipError_t launch_lmhead_kl_backward(const LMHeadShape& sh, const LMHeadShape& te, const float* lse_student,
                                     const float* lse_teacher, const float* grad_kl, float* grad_hidden,
                                     float* grad_weight, char* ws, const LMHeadWorkspace& w, hipStream_t s) {
  const bool fast = kl_fast_path(sh, te, 1) && (reinterpret_cast<uintptr_t>(grad_hidden) & 15u) == 0;
  float* tbuf = reinterpret_cast<float*>(ws + w.tbuf_off);
  auto launch_dz = [&](int64_t base, int64_t tr, int64_t tpad, int64_t vpad, int n_vb, int n_nb, const int* idx,
                       const int* count, uint16_t* dz, uint16_t* dzt) -> hipError_t {
    KLDzArgs d;
    d.h = kl_args(sh, te);
    d.h.idx = idx;
    d.h.count = count;
    d.h.targets = nullptr;
    d.h.n_vb = n_vb;
    d.h.part = nullptr;
    d.h.zy = nullptr;
    d.h.tbuf = tbuf;
    d.vpad = vpad;
    d.lse_u = lse_student;
    d.lse_v = lse_teacher;
    d.g = grad_kl;
    d.tpad = tpad;
    if (!fast) {
      d.h.tile_base = base;
      d.h.tile_rows = static_cast<int>(tr);
      d.h.n_nb = n_nb;
      d.dz = dz;
      d.dzt = dzt;
      TimedLaunch tl("k_kl_dz", s);
      hipLaunchKernelGGL(k_kl_dz<BwdCfg>, dim3(static_cast<unsigned>(n_vb) * n_nb), dim3(BwdCfg::NT), 0, s, d);
      return hipGetLastError();
    }
    // chunks of the tile that fit the teacher buffer; each fills its rows of dZ (and dZ^T)
    for (int64_t c0 = 0; c0 < tr; c0 += kKLChunk) {
      const int64_t cr = tr - c0 < kKLChunk ? tr - c0 : kKLChunk;
      d.h.tile_base = base + c0;
      d.h.tile_rows = static_cast<int>(cr);
      d.h.n_nb = static_cast<int>((cr + KLCfg::BN - 1) / KLCfg::BN);
      d.dz = dz + c0 * vpad;
      d.dzt = dzt ? dzt + c0 : nullptr;
      const dim3 grid(static_cast<unsigned>(n_vb) * d.h.n_nb);
      {
        TimedLaunch tl("k_kl_teacher", s);
        hipLaunchKernelGGL(k_kl_teacher_dtl<KLCfg>, grid, dim3(KLCfg::NT), 0, s, d.h);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      {
        TimedLaunch tl("k_kl_dz", s);
        hipLaunchKernelGGL(k_kl_dz_student_dtl<KLCfg>, grid, dim3(KLCfg::NT), 0, s, d);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
  };
  return backward_tiles(sh, fast, KLCfg::BM, KLCfg::BN, grad_hidden, grad_weight, ws, w, s, launch_dz);
}

}  // namespace lp
