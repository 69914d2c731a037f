/*
 * lp.h -- C ABI of liblp.so: per-token log-probabilities, entropy and exact
 * full-vocabulary KL over a large vocabulary on MI355X (gfx950), computed a
 * chunk (or tile) of rows at a time, never materialising [rows x vocab] fp32
 * logits.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every tensor argument is a DEVICE pointer owned by the caller.
 *   The library never allocates or frees device memory; scratch comes from
 *   the caller's `workspace`, except for the no-alloc forward, whose static
 *   scratch array each GPU holds from the library's first use on it.  Inputs are read-only and are never
 *   modified (unlike an in-place cross-entropy).
 * Layout: row-major.  A [rows x cols] matrix has row r at base + r * ld
 *   elements, ld >= cols.  Targets are int64, one per row.  A mask is uint8,
 *   one per row, nonzero = the row is scored; NULL = every row is scored.
 * Alignment: every array is aligned to its element size (fp32 to 4 bytes,
 *   int64 and fp64 to 8, bf16/fp16 logits to 2), or the call returns
 *   LP_ERR_INVALID_ARGUMENT; the fused paths' bf16 hidden states and weights
 *   must be 16-byte aligned (LP_ERR_UNSUPPORTED otherwise) and a workspace
 *   256-byte aligned.
 * Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *   asynchronous on it; outputs are valid once the stream reaches the call.
 * Errors: every argument is checked on the host before anything is launched.
 *   A non-LP_OK return launches nothing and leaves every output untouched;
 *   lp_last_error() then holds a thread-local description.  No exception or
 *   abort crosses this ABI.  A failure reported by the HIP runtime while
 *   launching gives LP_ERR_HIP.
 * Outputs are fp32.  Rows that are not scored get 0 in every per-row output
 *   and their targets are never read.
 * Temperature: applied to the fp32 values after the exact upcast, and only
 *   when temperature > 0 and temperature != 1 (otherwise the scale is 1) --
 *   the upcast helper `_upcast_chunk_to_fp32` on the miles PR #2764 summary
 *   page (prhub.com.cn), sections "实现拆解" item 2 and "关键源码片段".
 *   NaN or infinite temperatures are rejected.
 * Targets: a scored row needs 0 <= target < V; otherwise its log-prob is NaN
 *   (no device-to-host check is made); its entropy is still computed.
 * Special values: -inf logits are zero-probability entries and add nothing to
 *   the entropy; a row containing NaN or +inf, or only -inf, gives NaN.
 */
#ifndef LP_H_
#define LP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lp_status {
  LP_OK = 0,
  LP_ERR_INVALID_ARGUMENT = 1,
  LP_ERR_UNSUPPORTED = 2,
  LP_ERR_WORKSPACE_TOO_SMALL = 3,
  LP_ERR_HIP = 4
} lp_status;

typedef enum lp_dtype { LP_BF16 = 0, LP_FP16 = 1, LP_FP32 = 2 } lp_dtype;

/* Library version (major * 10000 + minor * 100 + patch). */
int lp_version(void);

/* Static text for a status code ("LP_OK", ...); "unknown status" otherwise. */
const char* lp_status_string(int status);

/* Thread-local description of the last non-OK return on this thread ("" if none). */
const char* lp_last_error(void);

/*
 * Log-prob of the target and entropy of each scored row of model-precision
 * logits.
 *
 * Follows calculate_log_probs_and_entropy on the miles PR #2764 summary page,
 * "关键源码片段": the logits stay in model precision; each chunk of rows is
 * widened to fp32 (here: in registers, never stored), divided by the
 * temperature in fp32, and reduced to log softmax at the target and the
 * Shannon entropy (nats) of softmax(z / temperature) over all V entries.
 *
 * logits      [T x ld] of `dtype` (LP_BF16, LP_FP16 or LP_FP32), ld >= V.
 * targets     int64 [T].  mask: uint8 [T] or NULL.
 * temperature see the file header.
 * chunk_rows  the page's chunk size (<= 0: one chunk).  On the page it bounds
 *             the rows widened to an fp32 tensor at once; this kernel never
 *             forms such a tensor (each row is widened in registers), so the
 *             chunks of a call (chunk_rows rows each, a short last one: 5 rows
 *             in chunks of 2 -> 2, 2, 1) run back to back in one launch.
 *             Memory use and results do not depend on it, bit for bit.
 * logprob     fp32 [T] (required).  entropy: fp32 [T] or NULL.
 * T == 0 returns LP_OK without launching.  Needs no workspace.
 */
lp_status lp_logprobs_entropy(const void* logits, lp_dtype dtype, int64_t T, int64_t V, int64_t ld,
                              const int64_t* targets, const uint8_t* mask, float temperature,
                              int64_t chunk_rows, float* logprob, float* entropy, void* stream);

/*
 * Bytes of device workspace the fused LM-head calls need (256-byte aligned
 * base required).  backward = 0 for lp_lm_head_logprobs_entropy, 1 for the
 * backward.  Returns 0 for invalid sizes.
 */
size_t lp_lm_head_workspace_bytes(int64_t T, int64_t h, int64_t V, int64_t tile_rows, int backward);

/*
 * Which GEMM tiles a fused LM-head call of this shape runs on (host only; no
 * device access): 1 = the direct-to-LDS MFMA tiles, 0 = the generic tiles,
 * -1 = invalid sizes (T < 0, h or V outside 1..2^30, ld_h or ld_w < h,
 * tile_rows <= 0).  The fast tiles need h % 64 == 0 and address every operand
 * with 32-bit per-lane byte offsets, so they also need
 *   (T x ld_h + h) x 2 < 2^32        (any hidden row may be gathered),
 *   (256 x ld_w + h) x 2 < 2^32      (one 256-row weight block),
 * and for the backward (backward != 0), with vpad = V rounded up to 64,
 * tpad = min(tile_rows, T) rounded up to 64 and ks = vpad / 4 rounded up to 64,
 *   (256 x vpad + vpad) x 2 < 2^32     (256-row blocks of the dZ buffer),
 *   (ks x ld_w + 256) x 2 < 2^32       (the weight rows of one K range of the
 *                                       hidden-gradient GEMM),
 *   (tpad x vpad + 256) x 2 < 2^32, (tpad x h + 256) x 2 < 2^32
 *                                      (dZ and the tile's hidden rows as the
 *                                       weight-gradient GEMM's operands).
 * Shapes outside these run on the generic tiles, which use 64-bit
 * addressing; results are the same up to summation order.  The backward also
 * takes the generic tiles when grad_hidden is not 16-byte aligned.  The KL
 * through the heads uses the fast tiles when both heads qualify.
 */
int lp_lm_head_fast_tiles(int64_t T, int64_t h, int64_t V, int64_t ld_h, int64_t ld_w, int64_t tile_rows,
                          int backward);

/*
 * Fused LM head forward: log-prob and entropy of softmax(hidden @ weight^T /
 * temperature) without writing the logits.
 *
 * Follows the fused_lm_head backend of miles PR #4645, "How it works": the
 * scored rows are selected first (prompt rows are never multiplied by the
 * output weight), then processed `tile_rows` at a time; here each tile's
 * logits live only in MFMA accumulators (fp32, never rounded to bf16) and are
 * folded straight into per-row running max / sum / entropy terms.
 *
 * hidden      bf16 [T x ld_h], ld_h >= h.  weight: bf16 [V x ld_w], ld_w >= h.
 * targets     int64 [T].  mask: uint8 [T] or NULL.
 * tile_rows   scored rows per tile, required, > 0 (no hidden default).
 * logprob     fp32 [T] (required); entropy fp32 [T] or NULL; lse fp32 [T] or
 *             NULL: log-sum-exp of the tempered logits, saved for the backward.
 * workspace   >= lp_lm_head_workspace_bytes(T, h, V, tile_rows, 0) bytes.
 * Restrictions (LP_ERR_UNSUPPORTED): h % 8 != 0, ld_h % 8 != 0, ld_w % 8 != 0,
 *   misaligned (not 16-byte) hidden or weight pointers, and shapes for which
 *   one launch would exceed 2^32-1 work-items (about V x min(T, tile_rows)
 *   past 2^36; a smaller tile_rows avoids it).  The same holds for the
 *   backward and for the KL through the heads.
 */
lp_status lp_lm_head_logprobs_entropy(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                                      int64_t T, int64_t h, int64_t V, const int64_t* targets,
                                      const uint8_t* mask, float temperature, int64_t tile_rows,
                                      float* logprob, float* entropy, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * The fused LM-head forward above for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): same arguments and results (bit for bit) without the
 * workspace.  Its scratch is a static device array of
 * LP_NOALLOC_SCRATCH_BYTES bytes that every GPU the library runs on holds
 * until the process ends; the call itself allocates and frees nothing.
 * The scratch used is the calling thread's current device's; a non-NULL
 * stream must belong to that device (LP_ERR_INVALID_ARGUMENT otherwise).
 * Shapes whose lp_lm_head_workspace_bytes(T, h, V, tile_rows, 0) exceeds the
 * scratch are refused with LP_ERR_WORKSPACE_TOO_SMALL (a smaller tile_rows
 * shrinks it: at V = 151936, tile_rows <= 1024 fits for T up to about 500k).
 * All calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (different streams or threads) race and give undefined results; calls
 * ordered on one stream are safe.  The first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress).
 */
#define LP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

lp_status lp_lm_head_logprobs_entropy_noalloc(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                                              int64_t T, int64_t h, int64_t V, const int64_t* targets,
                                              const uint8_t* mask, float temperature, int64_t tile_rows,
                                              float* logprob, float* entropy, float* lse, void* stream);

/*
 * Backward of the fused LM head for the loss
 *   L = sum over scored rows t of grad_logprob[t] * logprob[t] + grad_entropy[t] * entropy[t].
 * Recompute-based, as miles PR #4645 "How it works" describes: each tile's
 * logits are rebuilt by the same GEMM, turned into dL/dlogits in the
 * epilogue, then multiplied back by the weight (hidden gradient) and by the
 * tile's hidden rows (weight gradient).
 *
 * lse, entropy  fp32 [T] as written by the forward (same inputs, temperature).
 * grad_logprob  fp32 [T] (required); grad_entropy fp32 [T] or NULL (= 0).
 * grad_hidden   fp32 [T x h] or NULL: OVERWRITTEN; unscored rows get 0.
 * grad_weight   fp32 [V x h] or NULL (frozen weight: that GEMM is skipped):
 *               OVERWRITTEN with the sum over all scored rows.
 * workspace     >= lp_lm_head_workspace_bytes(T, h, V, tile_rows, 1) bytes.
 * With no scored rows both gradients are zero-filled.
 */
lp_status lp_lm_head_logprobs_entropy_backward(const void* hidden, int64_t ld_h, const void* weight,
                                               int64_t ld_w, int64_t T, int64_t h, int64_t V,
                                               const int64_t* targets, const uint8_t* mask,
                                               float temperature, int64_t tile_rows, const float* lse,
                                               const float* entropy, const float* grad_logprob,
                                               const float* grad_entropy, float* grad_hidden,
                                               float* grad_weight, void* workspace, size_t workspace_bytes,
                                               void* stream);

/*
 * Exact full-vocabulary KL(teacher || student) per row, no temperature, in
 * one pass over both rows.  DeepSeek-V4 book ch.19 "RL / OPD 工程", 名词速通:
 * "不实例化 logits" and "TileLang KL Kernel" (exact student/teacher KL).
 *
 * student, teacher  [T x ld_s], [T x ld_t] of `dtype` (LP_BF16, LP_FP16 or LP_FP32).
 * kl                fp32 [T] (required), every row.
 * targets           int64 [T] or NULL.  When given, lp_student / lp_teacher
 *                   (fp32 [T] or NULL) receive log softmax at the target for
 *                   every row, and prob_diff (fp32 [T] or NULL) receives
 *                   diff_mask ? |exp(lp_student) - exp(lp_teacher)| : 0, the
 *                   per-token measure of the msprobe page
 *                   "逐Token级别的probs_diff监控", §3.2.  diff_mask NULL = all rows.
 *                   With targets NULL those three outputs must be NULL.
 * Accumulation is fp32 throughout, so fp16 rows whose plain sums overflow
 * stay finite.  Needs no workspace.
 */
lp_status lp_kl_full_vocab(const void* student, const void* teacher, lp_dtype dtype, int64_t T, int64_t V,
                           int64_t ld_s, int64_t ld_t, float* kl, const int64_t* targets,
                           const uint8_t* diff_mask, float* lp_student, float* lp_teacher, float* prob_diff,
                           void* stream);

/*
 * out[i] = mask[i] ? |exp(lp_a[i]) - exp(lp_b[i])| : 0 for i < n
 * (msprobe page "逐Token级别的probs_diff监控", §3.2; an all-zero mask gives an
 * all-zero result, as in its edge-case table).  mask NULL = all positions.
 * All arrays fp32 / uint8, device, length n.
 */
lp_status lp_prob_diff(const float* lp_a, const float* lp_b, const uint8_t* mask, int64_t n, float* out,
                       void* stream);

/*
 * K targets per row (miles PR #4645, "Scope": the fused log-prob op with K
 * targets per row that score centering trains on).  Same as the single-target
 * calls above with targets [T x K] (row-major, K contiguous), 1 <= K <= 64,
 * and logprob [T x K]: logprob[t][k] = log softmax(z_t / temperature)[targets[t][k]].
 * The backward's loss is sum over scored rows of
 *   sum_k grad_logprob[t][k] * logprob[t][k] + grad_entropy[t] * entropy[t],
 * with grad_logprob [T x K].  Workspace sizes are those of the K = 1 calls.
 */
lp_status lp_logprobs_entropy_k(const void* logits, lp_dtype dtype, int64_t T, int64_t V, int64_t ld,
                                const int64_t* targets, int64_t K, const uint8_t* mask, float temperature,
                                int64_t chunk_rows, float* logprob, float* entropy, void* stream);

lp_status lp_lm_head_logprobs_entropy_k(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                                        int64_t T, int64_t h, int64_t V, const int64_t* targets, int64_t K,
                                        const uint8_t* mask, float temperature, int64_t tile_rows, float* logprob,
                                        float* entropy, float* lse, void* workspace, size_t workspace_bytes,
                                        void* stream);

lp_status lp_lm_head_logprobs_entropy_backward_k(const void* hidden, int64_t ld_h, const void* weight,
                                                 int64_t ld_w, int64_t T, int64_t h, int64_t V,
                                                 const int64_t* targets, int64_t K, const uint8_t* mask,
                                                 float temperature, int64_t tile_rows, const float* lse,
                                                 const float* entropy, const float* grad_logprob,
                                                 const float* grad_entropy, float* grad_hidden, float* grad_weight,
                                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * KL(teacher || student) with both models' logits rebuilt from cached last
 * hidden states through their own output heads, never materialised
 * (DeepSeek-V4 book ch.19: 名词速通 "不实例化 logits" and §2 "Teacher
 * Scheduling" -- the teacher's last hidden state is cached and passed
 * through its prediction head when the KL is computed).
 *
 * For each row t with mask[t] != 0 (mask NULL = all rows):
 *   u = student_hidden[t] . student_weight^T,  v = teacher_hidden[t] . teacher_weight^T
 *   (bf16 operands, fp32 MFMA accumulation, never rounded), and
 *   kl[t] = sum_j p_v,j (log p_v,j - log p_u,j) with p = softmax (no temperature),
 *   lse_student[t] = logsumexp(u), lse_teacher[t] = logsumexp(v),
 *   lp_student[t] = log p_u(y_t), lp_teacher[t] = log p_v(y_t)  (targets != NULL),
 *   prob_diff[t] = |exp(lp_student) - exp(lp_teacher)| where diff_mask[t] != 0
 *   (diff_mask NULL = all), else 0.
 * Rows with mask 0 get 0 in every output and are never multiplied.
 *
 * Layouts: hiddens bf16 [T x ld_h*] with h_student / h_teacher used columns;
 * weights bf16 [V x ld_w*] (both heads share the vocabulary); every h and ld
 * a multiple of 8; hiddens and weights 16-byte aligned.  Outputs are fp32
 * [T]; kl is required, every other output may be NULL (lp_student,
 * lp_teacher and prob_diff need targets).  A target outside [0, V) gives NaN
 * in lp_student / lp_teacher / prob_diff of that row only.
 * Workspace: lp_lm_head_kl_workspace_bytes(T, h_student, V, tile_rows, 0)
 * bytes, 256-byte aligned, caller-owned; scratch only.  Besides per-row
 * partial states it holds the teacher's fp32 logits of one chunk of rows
 * (min(tile_rows, 4096) x V x 4 bytes, rounded up to whole 256 x 256 blocks);
 * only the row index list grows with T, and tile_rows trades it for speed.
 * Errors as for the other LM-head calls: all checks before any launch.
 */
size_t lp_lm_head_kl_workspace_bytes(int64_t T, int64_t h_student, int64_t V, int64_t tile_rows, int backward);

lp_status lp_lm_head_kl(const void* student_hidden, int64_t ld_hs, const void* student_weight, int64_t ld_ws,
                        int64_t h_student, const void* teacher_hidden, int64_t ld_ht, const void* teacher_weight,
                        int64_t ld_wt, int64_t h_teacher, int64_t T, int64_t V, const uint8_t* mask,
                        const int64_t* targets, const uint8_t* diff_mask, int64_t tile_rows, float* kl,
                        float* lp_student, float* lp_teacher, float* prob_diff, float* lse_student,
                        float* lse_teacher, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of sum_t grad_kl[t] * kl[t] with respect to the student only (the
 * teacher head is frozen: it is only loaded to rebuild logits):
 *   dL/du_t,j = grad_kl[t] (p_u,j - p_v,j), rows with mask 0 contribute 0,
 *   grad_hidden = dL/du . student_weight   fp32 [T x h_student] (NULL: skipped),
 *   grad_weight = dL/du^T . student_hidden fp32 [V x h_student] (NULL: frozen).
 * Both logit tiles are recomputed; lse_student / lse_teacher are the forward's.
 * Workspace: lp_lm_head_kl_workspace_bytes(T, h_student, V, tile_rows, 1)
 * (the log-prob backward's buffers plus the same teacher-logit chunk).
 * With T == 0, grad_weight (if given) is zero-filled.
 */
lp_status lp_lm_head_kl_backward(const void* student_hidden, int64_t ld_hs, const void* student_weight,
                                 int64_t ld_ws, int64_t h_student, const void* teacher_hidden, int64_t ld_ht,
                                 const void* teacher_weight, int64_t ld_wt, int64_t h_teacher, int64_t T, int64_t V,
                                 const uint8_t* mask, int64_t tile_rows, const float* lse_student,
                                 const float* lse_teacher, const float* grad_kl, float* grad_hidden,
                                 float* grad_weight, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Aggregates of the masked prob diff, the macro statistics the msprobe page
 * lists next to its per-token diff (§4.1): over positions with mask != 0
 * (mask NULL = all), with pa = exp(lp_a), pb = exp(lp_b), d = |pa - pb|:
 *   out[0] = count, out[1] = max d, out[2] = mean d, out[3] = std d
 *   (population), out[4] = Pearson correlation of pa and pb.
 * Sums are fp64 and reduced in a fixed order (bitwise reproducible).  With
 * count 0 every output is 0 except out[4] = NaN, which is also NaN when
 * either series has zero variance.  out: device double[5], 8-byte aligned.
 * workspace: >= lp_prob_diff_stats_workspace_bytes() bytes, 256-byte aligned.
 */
size_t lp_prob_diff_stats_workspace_bytes(void);
lp_status lp_prob_diff_stats(const float* lp_a, const float* lp_b, const uint8_t* mask, int64_t n, double* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-kernel timing (observability; not part of the method).  While enabled,
 * each library launch is bracketed by two HIP events recorded on its own
 * stream.  lp_timing_enable(1) clears earlier records and starts recording,
 * lp_timing_enable(0) clears and stops.  lp_timing_read() waits for the
 * recorded events of `kernel` (e.g. "k_fwd_tile", "k_logprobs_entropy",
 * "k_kl_full_vocab") and returns the number of launches and their summed
 * duration in milliseconds.  Records are process-wide and thread-safe.
 */
void lp_timing_enable(int on);
lp_status lp_timing_read(const char* kernel, int64_t* launches, double* total_ms);

/*
 * With lp_timing_enable(2) (timing plus clock samples), every workgroup of the
 * fused forward's MFMA kernel on the direct-to-LDS tiles also records the
 * deltas of the shader-clock counter and of the fixed-frequency counter over
 * its run (a static device array of 65536 sample pairs, overwritten by each
 * launch).  lp_timing_clock("k_fwd_tile", &mhz, &samples) waits for the
 * device and returns the mean shader clock (MHz) over the workgroups of the
 * last such launch that had work, and their number (0 if none).  Other
 * kernel names: LP_ERR_UNSUPPORTED.
 */
lp_status lp_timing_clock(const char* kernel, double* mhz, int64_t* samples);

#ifdef __cplusplus
}
#endif

#endif /* LP_H_ */
