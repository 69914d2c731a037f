"""Plain fp64 CPU oracle for per-token log-probs, entropy, exact full-vocab KL
and the masked probability diff.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, the smoke check and the benchmark's CPU-baseline leg call it.  It
shares no code, tables or constants with the HIP path.

Every function materialises the full logits of the rows it is given (in fp64)
and applies the textbook definition.  The chunked / fused method reaches the
same numbers up to rounding order, so the definition *is* the oracle:

* upcast before temperature: the miles PR #2764 summary (prhub.com.cn),
  sections "实现拆解" item 2 and "关键源码片段" (`_upcast_chunk_to_fp32`):
  the chunk is widened to fp32 first and divided by the temperature only when
  the temperature is positive and not 1.  Here the widening is exact (fp64).
* log-prob of the target and entropy of each row: same page, "实现拆解" item 2
  (entropy goes through the same upcast helper) and "关键源码片段"
  (`calculate_log_probs_and_entropy`).
* rows that are not scored give 0: msprobe "逐Token级别的probs_diff监控"
  page, §4.3.1 (padding positions hold 0), and miles PR #4645 "How it works"
  (prompt rows are never multiplied by the output weight).
* fused LM head: miles PR #4645, "How it works": the logits of a scored row
  are the output layer applied to its hidden state, hidden @ W^T.
* backward: miles PR #4645, "How it works" (the backward replays the tile and
  produces hidden and weight gradients) and "Testing" (equality of the
  hidden/weight gradients against hidden @ W^T).
* exact KL between teacher and student over the whole vocabulary:
  DeepSeek-V4 book ch.19 "RL / OPD 工程", 名词速通 "不实例化 logits" and
  "TileLang KL Kernel".
* masked |exp(lp_a) - exp(lp_b)|: msprobe page §3.2
  (`calculate_token_level_prob_diff`) and its edge-case table; its
  aggregates (max / mean / std / Pearson): same page §4.1.
* K target ids per row: miles PR #4645 "Scope" (the fused op with K targets
  per row that score centering trains on).
* KL with each model's logits rebuilt from its cached last hidden state
  through its own output head: DeepSeek-V4 book ch.19, 名词速通
  "不实例化 logits" and §2 "Teacher Scheduling".

Where the pages are silent, the reading taken is stated next to the code
that takes it.
"""
from __future__ import annotations

import numpy as np

LN2 = float(np.log(2.0))


# ---------------------------------------------------------------------------
# exact widening of model-precision bits
# ---------------------------------------------------------------------------

def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64, exactly (bf16 is the top half of fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def widen_fp16(bits) -> np.ndarray:
    """fp16 bit patterns (uint16) -> fp64, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return b.view(np.float16).astype(np.float64)


def widen(bits, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return widen_bf16(bits)
    if dtype == "fp16":
        return widen_fp16(bits)
    if dtype == "fp32":
        return np.ascontiguousarray(bits, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# temperature (miles PR #2764 summary, `_upcast_chunk_to_fp32`)
# ---------------------------------------------------------------------------

def temperature_applies(temperature: float) -> bool:
    """The helper divides only when the temperature is > 0 and != 1."""
    return bool(temperature > 0.0 and temperature != 1.0)


def tempered(z: np.ndarray, temperature: float) -> np.ndarray:
    """z / temperature after the (already exact) upcast, else z unchanged."""
    z = np.asarray(z, dtype=np.float64)
    if temperature_applies(temperature):
        return z / np.float64(temperature)
    return z.copy()


# ---------------------------------------------------------------------------
# textbook log-softmax pieces
# ---------------------------------------------------------------------------

def log_normaliser(zt: np.ndarray) -> np.ndarray:
    """log sum_j exp(zt_j) per row, with the usual max shift.

    Rows whose entries are all -inf give -inf.
    """
    zt = np.atleast_2d(np.asarray(zt, dtype=np.float64))
    m = zt.max(axis=1)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(under="ignore", invalid="ignore"):
        s = np.exp(zt - safe_m[:, None]).sum(axis=1)
        return safe_m + np.log(s)


def log_softmax(zt: np.ndarray) -> np.ndarray:
    zt = np.atleast_2d(np.asarray(zt, dtype=np.float64))
    return zt - log_normaliser(zt)[:, None]


def shannon_entropy(logp: np.ndarray) -> np.ndarray:
    """-sum_j p_j log p_j in nats, with 0 log 0 = 0 (so -inf logits add nothing)."""
    with np.errstate(under="ignore", invalid="ignore"):
        p = np.exp(logp)
        terms = np.where(p > 0.0, p * logp, 0.0)
    return -terms.sum(axis=1)


def _scored(mask, T: int) -> np.ndarray:
    if mask is None:
        return np.ones(T, dtype=bool)
    return np.asarray(mask).reshape(T) != 0


def _gather_targets(logp: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """logp[t, y_t]; a target outside [0, V) gives NaN (reading: poison, no raise)."""
    T, V = logp.shape
    y = np.asarray(targets, dtype=np.int64).reshape(T)
    ok = (y >= 0) & (y < V)
    out = np.full(T, np.nan)
    rows = np.nonzero(ok)[0]
    out[rows] = logp[rows, y[rows]]
    return out


# ---------------------------------------------------------------------------
# logits-input path
# ---------------------------------------------------------------------------

def logprobs_entropy(logits: np.ndarray, targets, mask, temperature: float):
    """Per-row log p(target) and entropy of softmax(logits / temperature).

    `logits` are the widened model-precision values, shape [T, V].
    Returns (logprob[T], entropy[T], lse[T]) in fp64; unscored rows are 0.
    `lse` is log sum exp of the tempered logits (0 on unscored rows).
    """
    z = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    T = z.shape[0]
    keep = _scored(mask, T)
    lp = np.zeros(T)
    H = np.zeros(T)
    lse = np.zeros(T)
    if T == 0 or not keep.any():
        return lp, H, lse
    rows = np.nonzero(keep)[0]
    zt = tempered(z[rows], temperature)
    norm = log_normaliser(zt)
    logp = zt - norm[:, None]
    lp[rows] = _gather_targets(logp, np.asarray(targets).reshape(T)[rows])
    H[rows] = shannon_entropy(logp)
    lse[rows] = norm
    return lp, H, lse


def chunk_plan(T: int, chunk_rows: int):
    """Row ranges processed one launch at a time.

    Reading: fixed-size chunks of `chunk_rows` with a short last chunk (the
    page's own example of 5 rows in chunks of 2 gives sizes 2, 2, 1); a
    non-positive chunk size means one chunk of all rows.  Results never
    depend on the plan.
    """
    if T <= 0:
        return []
    if chunk_rows <= 0 or chunk_rows >= T:
        return [(0, T)]
    return [(s, min(chunk_rows, T - s)) for s in range(0, T, chunk_rows)]


# ---------------------------------------------------------------------------
# fused LM head (miles PR #4645, "How it works")
# ---------------------------------------------------------------------------

def lm_head_logits(hidden: np.ndarray, weight: np.ndarray, vocab_block: int = 16384) -> np.ndarray:
    """Z = hidden @ weight^T in fp64.

    Products of bf16 values are exact in fp64.  The vocabulary is walked in
    column blocks only so that `weight` never has to be widened in one piece;
    every entry of Z is the same fp64 dot product either way.
    """
    Hd = np.asarray(hidden, dtype=np.float64)
    T = Hd.shape[0]
    V = weight.shape[0]
    Z = np.empty((T, V))
    for j0 in range(0, V, vocab_block):
        j1 = min(V, j0 + vocab_block)
        Wb = np.asarray(weight[j0:j1], dtype=np.float64)
        Z[:, j0:j1] = Hd @ Wb.T
    return Z


def lm_head_logprobs_entropy(hidden, weight, targets, mask, temperature: float):
    """Forward of the fused LM head on widened hidden [T, h] and weight [V, h].

    Returns (logprob, entropy, lse), unscored rows 0.  Only scored rows are
    multiplied by the weight.
    """
    hidden = np.atleast_2d(np.asarray(hidden, dtype=np.float64))
    T = hidden.shape[0]
    keep = _scored(mask, T)
    lp = np.zeros(T)
    H = np.zeros(T)
    lse = np.zeros(T)
    rows = np.nonzero(keep)[0]
    if rows.size == 0:
        return lp, H, lse
    Z = lm_head_logits(hidden[rows], weight)
    sub_lp, sub_H, sub_lse = logprobs_entropy(Z, np.asarray(targets).reshape(T)[rows], None, temperature)
    lp[rows] = sub_lp
    H[rows] = sub_H
    lse[rows] = sub_lse
    return lp, H, lse


def lm_head_loss(hidden, weight, targets, mask, temperature, grad_logprob, grad_entropy) -> float:
    """The scalar whose gradient the backward returns: sum_t g_lp,t lp_t + g_H,t H_t."""
    lp, H, _ = lm_head_logprobs_entropy(hidden, weight, targets, mask, temperature)
    T = lp.shape[0]
    keep = _scored(mask, T)
    g_lp = np.asarray(grad_logprob, dtype=np.float64).reshape(T)
    g_H = np.zeros(T) if grad_entropy is None else np.asarray(grad_entropy, dtype=np.float64).reshape(T)
    return float(np.sum(np.where(keep, g_lp * lp + g_H * H, 0.0)))


def lm_head_logit_grad(hidden, weight, targets, mask, temperature, grad_logprob, grad_entropy):
    """dL/dZ for the scored rows (chain rule through log-softmax and entropy).

    With zt = Z / tau (tau applied as in the upcast helper) and
    logp = log_softmax(zt):
      d lp_t / d zt_tj = [j == y_t] - p_tj
      d H_t  / d zt_tj = -p_tj (logp_tj + H_t)
    and dZ = dzt / tau.  Unscored rows get 0.
    Returns (rows, dZ[rows]) so callers can form either gradient.
    """
    hidden = np.atleast_2d(np.asarray(hidden, dtype=np.float64))
    T = hidden.shape[0]
    keep = _scored(mask, T)
    rows = np.nonzero(keep)[0]
    V = weight.shape[0]
    if rows.size == 0:
        return rows, np.zeros((0, V))
    Z = lm_head_logits(hidden[rows], weight)
    zt = tempered(Z, temperature)
    logp = log_softmax(zt)
    p = np.exp(logp)
    Hrow = shannon_entropy(logp)
    y = np.asarray(targets, dtype=np.int64).reshape(T)[rows]
    g_lp = np.asarray(grad_logprob, dtype=np.float64).reshape(T)[rows]
    g_H = (np.zeros(rows.size) if grad_entropy is None
           else np.asarray(grad_entropy, dtype=np.float64).reshape(T)[rows])
    onehot = np.zeros_like(p)
    onehot[np.arange(rows.size), y] = 1.0
    with np.errstate(invalid="ignore"):
        plogp_shift = np.where(p > 0.0, p * (logp + Hrow[:, None]), 0.0)
    dzt = g_lp[:, None] * (onehot - p) - g_H[:, None] * plogp_shift
    scale = (1.0 / temperature) if temperature_applies(temperature) else 1.0
    return rows, dzt * scale


def lm_head_backward(hidden, weight, targets, mask, temperature, grad_logprob, grad_entropy):
    """(dHidden [T, h], dWeight [V, h]) in fp64 for the loss of `lm_head_loss`.

    dHidden = dZ @ W (zero on unscored rows), dWeight = dZ^T @ hidden.
    """
    hidden = np.atleast_2d(np.asarray(hidden, dtype=np.float64))
    T, h = hidden.shape
    W = np.asarray(weight, dtype=np.float64)
    rows, dZ = lm_head_logit_grad(hidden, weight, targets, mask, temperature, grad_logprob, grad_entropy)
    dH = np.zeros((T, h))
    dW = np.zeros(W.shape)
    if rows.size:
        dH[rows] = dZ @ W
        dW = dZ.T @ hidden[rows]
    return dH, dW


# ---------------------------------------------------------------------------
# exact full-vocab KL and the prob diff
# ---------------------------------------------------------------------------

def kl_full_vocab(student: np.ndarray, teacher: np.ndarray) -> np.ndarray:
    """KL(teacher || student) per row over the whole vocabulary, no temperature.

    KL = sum_j p_teacher,j (log p_teacher,j - log p_student,j), 0 log 0 = 0.
    """
    u = np.atleast_2d(np.asarray(student, dtype=np.float64))
    v = np.atleast_2d(np.asarray(teacher, dtype=np.float64))
    lpu = log_softmax(u)
    lpv = log_softmax(v)
    with np.errstate(under="ignore", invalid="ignore"):
        pv = np.exp(lpv)
        terms = np.where(pv > 0.0, pv * (lpv - lpu), 0.0)
    return terms.sum(axis=1)


def target_logprobs(logits: np.ndarray, targets) -> np.ndarray:
    """log softmax(logits)[t, y_t] with no temperature (all rows)."""
    z = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    return _gather_targets(log_softmax(z), targets)


def prob_diff(lp_a, lp_b, mask) -> np.ndarray:
    """mask * |exp(lp_a) - exp(lp_b)|  (msprobe page, §3.2).  mask None = all."""
    a = np.asarray(lp_a, dtype=np.float64)
    b = np.asarray(lp_b, dtype=np.float64)
    d = np.abs(np.exp(a) - np.exp(b))
    if mask is None:
        return d
    keep = np.asarray(mask).reshape(a.shape) != 0
    return np.where(keep, d, 0.0)


def kl_and_prob_diff(student, teacher, targets, diff_mask):
    """Everything the KL entry point returns, for the rows given.

    Returns (kl, lp_student, lp_teacher, diff): lp_* are the target log-probs
    of each model, diff = mask * |exp(lp_student) - exp(lp_teacher)|.
    """
    kl = kl_full_vocab(student, teacher)
    lpu = target_logprobs(student, targets)
    lpv = target_logprobs(teacher, targets)
    return kl, lpu, lpv, prob_diff(lpu, lpv, diff_mask)


# ---------------------------------------------------------------------------
# aggregates of the prob diff (msprobe page §4.1: max / mean / std of the
# masked diff and the Pearson correlation of the two probability series)
# ---------------------------------------------------------------------------

def prob_diff_stats(lp_a, lp_b, mask):
    """(count, max, mean, std, pearson) over positions with mask != 0.

    diff = |exp(lp_a) - exp(lp_b)|; std is the population std (ddof 0, as
    numpy's default in the page's offline example); pearson is the
    correlation of exp(lp_a) and exp(lp_b).  Reading: with no masked
    position every statistic is 0 except pearson, which is NaN, as it is
    when either series has zero variance.
    """
    a = np.asarray(lp_a, dtype=np.float64).ravel()
    b = np.asarray(lp_b, dtype=np.float64).ravel()
    keep = np.ones(a.shape, bool) if mask is None else (np.asarray(mask).ravel() != 0)
    pa, pb = np.exp(a[keep]), np.exp(b[keep])
    n = int(keep.sum())
    if n == 0:
        return 0, 0.0, 0.0, 0.0, float("nan")
    d = np.abs(pa - pb)
    sa, sb = pa.std(), pb.std()
    if sa == 0.0 or sb == 0.0:
        r = float("nan")
    else:
        r = float(np.mean((pa - pa.mean()) * (pb - pb.mean())) / (sa * sb))
    return n, float(d.max()), float(d.mean()), float(d.std()), r


# ---------------------------------------------------------------------------
# K targets per row (miles PR #4645, "Scope": the fused log-prob op with K
# targets per row that score centering trains on)
# ---------------------------------------------------------------------------

def logprobs_entropy_k(logits, targets_k, mask, temperature: float):
    """log softmax(z / tau) at each of K targets per row: (logprob[T, K], entropy[T], lse[T])."""
    z = np.atleast_2d(np.asarray(logits, dtype=np.float64))
    T = z.shape[0]
    y = np.asarray(targets_k, dtype=np.int64).reshape(T, -1)
    K = y.shape[1]
    keep = _scored(mask, T)
    lp = np.zeros((T, K))
    H = np.zeros(T)
    lse = np.zeros(T)
    rows = np.nonzero(keep)[0]
    if rows.size == 0:
        return lp, H, lse
    zt = tempered(z[rows], temperature)
    norm = log_normaliser(zt)
    logp = zt - norm[:, None]
    for k in range(K):
        lp[rows, k] = _gather_targets(logp, y[rows, k])
    H[rows] = shannon_entropy(logp)
    lse[rows] = norm
    return lp, H, lse


def lm_head_logprobs_entropy_k(hidden, weight, targets_k, mask, temperature: float):
    hidden = np.atleast_2d(np.asarray(hidden, dtype=np.float64))
    T = hidden.shape[0]
    y = np.asarray(targets_k, dtype=np.int64).reshape(T, -1)
    keep = _scored(mask, T)
    rows = np.nonzero(keep)[0]
    lp = np.zeros((T, y.shape[1]))
    H = np.zeros(T)
    lse = np.zeros(T)
    if rows.size == 0:
        return lp, H, lse
    Z = lm_head_logits(hidden[rows], weight)
    sub = logprobs_entropy_k(Z, y[rows], None, temperature)
    lp[rows], H[rows], lse[rows] = sub
    return lp, H, lse


def lm_head_loss_k(hidden, weight, targets_k, mask, temperature, grad_logprob_k, grad_entropy) -> float:
    """sum over scored rows of sum_k g_lp[t, k] lp[t, k] + g_H[t] H[t]."""
    lp, H, _ = lm_head_logprobs_entropy_k(hidden, weight, targets_k, mask, temperature)
    T = lp.shape[0]
    keep = _scored(mask, T)
    g = np.asarray(grad_logprob_k, dtype=np.float64).reshape(lp.shape)
    gH = np.zeros(T) if grad_entropy is None else np.asarray(grad_entropy, dtype=np.float64).reshape(T)
    return float(np.sum(np.where(keep, (g * lp).sum(axis=1) + gH * H, 0.0)))


def lm_head_backward_k(hidden, weight, targets_k, mask, temperature, grad_logprob_k, grad_entropy):
    """(dHidden, dWeight) of `lm_head_loss_k`: with zt = Z / tau and logp = log_softmax(zt),
      d lp_tk / d zt_tj = [j == y_tk] - p_tj,   d H_t / d zt_tj = -p_tj (logp_tj + H_t),
    summed with the weights g_lp[t, k] and g_H[t], then dZ = dzt / tau."""
    hidden = np.atleast_2d(np.asarray(hidden, dtype=np.float64))
    T, h = hidden.shape
    W = np.asarray(weight, dtype=np.float64)
    y = np.asarray(targets_k, dtype=np.int64).reshape(T, -1)
    g = np.asarray(grad_logprob_k, dtype=np.float64).reshape(y.shape)
    gH = np.zeros(T) if grad_entropy is None else np.asarray(grad_entropy, dtype=np.float64).reshape(T)
    rows = np.nonzero(_scored(mask, T))[0]
    dH = np.zeros((T, h))
    dW = np.zeros(W.shape)
    if rows.size == 0:
        return dH, dW
    zt = tempered(lm_head_logits(hidden[rows], W), temperature)
    logp = log_softmax(zt)
    p = np.exp(logp)
    Hrow = shannon_entropy(logp)
    dzt = -g[rows].sum(axis=1)[:, None] * p
    for k in range(y.shape[1]):
        np.add.at(dzt, (np.arange(rows.size), y[rows, k]), g[rows, k])
    with np.errstate(invalid="ignore"):
        dzt -= gH[rows][:, None] * np.where(p > 0.0, p * (logp + Hrow[:, None]), 0.0)
    dZ = dzt * ((1.0 / temperature) if temperature_applies(temperature) else 1.0)
    dH[rows] = dZ @ W
    dW = dZ.T @ hidden[rows]
    return dH, dW


# ---------------------------------------------------------------------------
# KL rebuilt from cached hidden states through each model's output head
# (DeepSeek-V4 book ch.19 "RL / OPD 工程": 名词速通 "不实例化 logits" and
# §2 "Teacher Scheduling": only the last hidden state is kept and the logits
# are rebuilt through the matching prediction head when the KL is computed)
# ---------------------------------------------------------------------------

def lm_head_kl(hidden_s, weight_s, hidden_t, weight_t, mask, targets, diff_mask):
    """KL(teacher || student) of the rows' logits hidden @ W^T of each model.

    Returns (kl, lp_student, lp_teacher, diff, lse_student, lse_teacher), each
    [T]; rows with mask == 0 are 0 everywhere.  No temperature, as for the KL
    on given logits.  targets None: lp_*, diff are all 0.  diff is
    |exp(lp_student) - exp(lp_teacher)| on scored rows whose diff_mask is set.
    """
    hs = np.atleast_2d(np.asarray(hidden_s, dtype=np.float64))
    ht = np.atleast_2d(np.asarray(hidden_t, dtype=np.float64))
    T = hs.shape[0]
    out = [np.zeros(T) for _ in range(6)]
    rows = np.nonzero(_scored(mask, T))[0]
    if rows.size == 0:
        return tuple(out)
    u = lm_head_logits(hs[rows], weight_s)
    v = lm_head_logits(ht[rows], weight_t)
    out[0][rows] = kl_full_vocab(u, v)
    out[4][rows] = log_normaliser(u)
    out[5][rows] = log_normaliser(v)
    if targets is not None:
        y = np.asarray(targets, dtype=np.int64).reshape(T)[rows]
        out[1][rows] = target_logprobs(u, y)
        out[2][rows] = target_logprobs(v, y)
        dm = None if diff_mask is None else np.asarray(diff_mask).reshape(T)[rows]
        out[3][rows] = prob_diff(out[1][rows], out[2][rows], dm)
    return tuple(out)


def lm_head_kl_loss(hidden_s, weight_s, hidden_t, weight_t, mask, grad_kl) -> float:
    """sum over scored rows of g_t KL_t (the scalar the KL backward differentiates)."""
    kl = lm_head_kl(hidden_s, weight_s, hidden_t, weight_t, mask, None, None)[0]
    return float(np.dot(np.asarray(grad_kl, dtype=np.float64).reshape(kl.shape), kl))


def lm_head_kl_logit_grad(hidden_s, weight_s, hidden_t, weight_t, mask, grad_kl):
    """(scored rows, dL/du [rows, V]) for the loss sum_t g_t KL_t.

    KL_t = sum_j p_v (log p_v - log p_u) depends on the student logits u only
    through -sum_j p_v log p_u = lse_u - sum_j p_v u_j, whose derivative in
    u_j is p_u,j - p_v,j.
    """
    hs = np.atleast_2d(np.asarray(hidden_s, dtype=np.float64))
    ht = np.atleast_2d(np.asarray(hidden_t, dtype=np.float64))
    T = hs.shape[0]
    g = np.asarray(grad_kl, dtype=np.float64).reshape(T)
    rows = np.nonzero(_scored(mask, T))[0]
    if rows.size == 0:
        return rows, np.zeros((0, weight_s.shape[0]))
    pu = np.exp(log_softmax(lm_head_logits(hs[rows], weight_s)))
    pv = np.exp(log_softmax(lm_head_logits(ht[rows], weight_t)))
    return rows, g[rows][:, None] * (pu - pv)


def lm_head_kl_backward(hidden_s, weight_s, hidden_t, weight_t, mask, grad_kl):
    """(dHidden_student, dWeight_student) of `lm_head_kl_loss`: dH = dZ . W_s,
    dW = dZ^T . H_s with dZ from `lm_head_kl_logit_grad`.  The teacher is not
    trained (its head is only loaded to rebuild logits), so no teacher
    gradient is formed."""
    hs = np.atleast_2d(np.asarray(hidden_s, dtype=np.float64))
    T, h = hs.shape
    Ws = np.asarray(weight_s, dtype=np.float64)
    dH = np.zeros((T, h))
    dW = np.zeros(Ws.shape)
    rows, dZ = lm_head_kl_logit_grad(hs, Ws, hidden_t, weight_t, mask, grad_kl)
    if rows.size == 0:
        return dH, dW
    dH[rows] = dZ @ Ws
    dW = dZ.T @ hs[rows]
    return dH, dW
