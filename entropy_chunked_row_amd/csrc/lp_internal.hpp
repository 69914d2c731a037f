// Internal interface between the C-ABI host layer (lp_api.cpp) and the kernel
// translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lp {

// Most targets per row the K-target entry points accept.
constexpr int kMaxTargets = 64;

// RAII bracket around one kernel launch: records HIP events on the launch
// stream when timing is enabled (lp_timing_enable), else does nothing.
class TimedLaunch {
 public:
  TimedLaunch(const char* name, hipStream_t s);
  ~TimedLaunch();
  TimedLaunch(const TimedLaunch&) = delete;
  TimedLaunch& operator=(const TimedLaunch&) = delete;

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_;
};

// True while lp_timing_enable(2) is in force: the fast forward GEMM then also
// records, per workgroup, the shader-clock and fixed-frequency counter deltas
// of its run (read back by lp_timing_clock).
bool timing_clocks_on();

// Copies the per-workgroup clock samples of the last fast forward launch made
// while timing_clocks_on(): pairs (shader-clock delta, fixed-clock delta) for
// its first *n workgroups (*n = at most the samples held; 0 if none).
hipError_t read_fwd_clocks(unsigned long long* pairs, int64_t* n);

// Logits-input rows [row0, row0 + rows) of a [T x ld] matrix.
struct RowArgs {
  const void* x;
  int64_t ld;
  int V;
  int64_t row0;
  int64_t rows;
  const int64_t* targets;  // [T x K]
  int K;                   // targets per row
  const uint8_t* mask;
  float c;  // log2(e) / tau_effective, rounded once on the host
  float* logprob;          // [T x K]
  float* entropy;
};

struct KLArgs {
  const void* student;
  const void* teacher;
  int64_t ld_s, ld_t;
  int V;
  int64_t T;
  int64_t row0;  // first row of the launch (set by the launcher)
  float c;  // log2(e)
  float* kl;
  const int64_t* targets;
  const uint8_t* diff_mask;
  float* lp_student;
  float* lp_teacher;
  float* prob_diff;
};

hipError_t launch_logprobs_entropy(int dtype, const RowArgs& a, hipStream_t s);
hipError_t launch_kl_full_vocab(int dtype, const KLArgs& a, hipStream_t s);
hipError_t launch_prob_diff(const float* a, const float* b, const uint8_t* mask, int64_t n, float* out,
                            hipStream_t s);

// Aggregates of the masked prob diff: out[0..4] = count, max, mean, std, pearson.
size_t prob_diff_stats_workspace_bytes();
hipError_t launch_prob_diff_stats(const float* a, const float* b, const uint8_t* mask, int64_t n, double* out,
                                  void* ws, hipStream_t s);

// ---------------------------------------------------------------------------
// fused LM head
// ---------------------------------------------------------------------------

struct LMHeadShape {
  const uint16_t* hidden;  // bf16 bits [T x ld_h]
  int64_t ld_h;
  const uint16_t* weight;  // bf16 bits [V x ld_w]
  int64_t ld_w;
  int64_t T;
  int h;
  int V;
  const int64_t* targets;  // [T x K]
  int K;                   // targets per row (1 .. kMaxTargets)
  const uint8_t* mask;
  float c;        // log2(e) / tau_effective
  float inv_tau;  // 1 / tau_effective
  int64_t tile_rows;
};

// Workspace carve-up shared by forward and backward (offsets in bytes from the
// 256-byte aligned base).
struct LMHeadWorkspace {
  size_t idx_off;     // int32 [T]      scored-row indices, ascending
  size_t count_off;   // int32 [1]      number of scored rows
  size_t part_off;    // float [tile_rows x n_vblocks x 3]   (forward)
  size_t zy_off;      // float [tile_rows]                   (forward)
  size_t dz_off;      // bf16 [tile_rows x Vpad]             (backward)
  size_t tbuf_off;    // float teacher logits of one row chunk (KL, direct-to-LDS tiles)
  size_t total;
  int n_vblocks;
  int64_t vpad;
};

// backward: 0 log-prob forward, 1 log-prob backward, 2 KL forward, 3 KL backward.
bool lmhead_workspace_layout(int64_t T, int64_t h, int64_t V, int64_t tile_rows, int backward,
                             LMHeadWorkspace* w);

// False when some launch of the call would exceed 2^32 - 1 work-items (a
// smaller tile_rows fixes it); same modes as lmhead_workspace_layout.
bool lmhead_launches_fit(int64_t T, int64_t h, int64_t V, int64_t tile_rows, int backward);

// True when a call of this shape runs on the direct-to-LDS tiles (every
// per-lane byte offset of their loads fits in 32 bits and h % 64 == 0);
// backward: also the dense gradient GEMMs on the dZ buffers.  Otherwise the
// generic tiles (64-bit addressing) run.
bool lmhead_fast_tiles(int64_t T, int64_t h, int64_t V, int64_t ld_h, int64_t ld_w, int64_t tile_rows, int backward);

// Zero-fill with a kernel (not a memset node, so callers may capture it).
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);

hipError_t launch_lmhead_forward(const LMHeadShape& sh, float* logprob, float* entropy, float* lse,
                                 char* ws, const LMHeadWorkspace& w, hipStream_t s);

hipError_t launch_lmhead_backward(const LMHeadShape& sh, const float* lse, const float* entropy,
                                  const float* grad_logprob, const float* grad_entropy, float* grad_hidden,
                                  float* grad_weight, char* ws, const LMHeadWorkspace& w, hipStream_t s);

// KL(teacher || student) with both models' logits rebuilt through their heads.
// `student` carries the student's hidden / weight / h plus T, V, mask and
// tile_rows; `teacher` its hidden / weight / h (other fields unused).
struct KLHeadOutputs {
  float* kl;
  float* lp_student;
  float* lp_teacher;
  float* prob_diff;
  float* lse_student;
  float* lse_teacher;
};

hipError_t launch_lmhead_kl_forward(const LMHeadShape& student, const LMHeadShape& teacher, const int64_t* targets,
                                    const uint8_t* diff_mask, const KLHeadOutputs& out, char* ws,
                                    const LMHeadWorkspace& w, hipStream_t s);

hipError_t launch_lmhead_kl_backward(const LMHeadShape& student, const LMHeadShape& teacher, const float* lse_student,
                                     const float* lse_teacher, const float* grad_kl, float* grad_hidden,
                                     float* grad_weight, char* ws, const LMHeadWorkspace& w, hipStream_t s);

}  // namespace lp
