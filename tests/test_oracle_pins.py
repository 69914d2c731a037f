"""Pins for the fp64 oracle: closed forms, brute force, finite differences,
invariants and the pages' own worked example.  None of these re-types the
oracle's formulas; each checks it against something the pages or the
mathematics fix independently.  Mutation tests at the end plant plausible
mistakes in the oracle (on the CPU) and check that a pin catches each one.
"""
import math
import os

import numpy as np
import pytest

import oracle.lp_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent brute-force formulations (pure Python, math.fsum, no max shift)
# ---------------------------------------------------------------------------

def bf_row(z, y, tau):
    """softmax by direct exp / fsum on a safe range; returns (lp_y, entropy)."""
    scale = (1.0 / tau) if (tau > 0 and tau != 1.0) else 1.0
    e = [math.exp(float(v) * scale) for v in z]
    S = math.fsum(e)
    p = [x / S for x in e]
    H = -math.fsum(pi * math.log(pi) for pi in p if pi > 0)
    return math.log(p[y]), H


def bf_kl(u, v):
    eu = [math.exp(float(x)) for x in u]
    ev = [math.exp(float(x)) for x in v]
    Su, Sv = math.fsum(eu), math.fsum(ev)
    return math.fsum((b / Sv) * math.log((b / Sv) / (a / Su)) for a, b in zip(eu, ev))


def bf_matmul_T(Hm, Wm):
    T, h = len(Hm), len(Hm[0])
    V = len(Wm)
    return [[math.fsum(Hm[t][k] * Wm[j][k] for k in range(h)) for j in range(V)] for t in range(T)]


# ---------------------------------------------------------------------------
# pins: logits-input path
# ---------------------------------------------------------------------------

def pin_uniform():
    for V in (1, 2, 7, 1000, 151936):
        for c in (0.0, -3.5, 12.25):
            for tau in (1.0, 0.7, 2.0):
                lp, H, _ = O.logprobs_entropy(np.full((1, V), c), [V - 1], None, tau)
                assert abs(lp[0] + math.log(V)) < 1e-12 * max(1, math.log(V))
                assert abs(H[0] - math.log(V)) < 1e-12 * max(1, math.log(V))


def test_uniform_rows_closed_form():
    pin_uniform()


def test_single_class():
    lp, H, _ = O.logprobs_entropy(np.array([[3.25], [-7.0]]), [0, 0], None, 0.7)
    assert np.all(lp == 0.0) and np.all(H == 0.0)


def pin_two_class():
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.normal(0, 3, size=2)
        y = int(rng.integers(0, 2))
        tau = float(rng.choice([0.7, 1.0, 1.9]))
        d = (z[1 - y] - z[y]) / tau
        lp_ref = -math.log1p(math.exp(d))          # -softplus(d)
        q = 1.0 / (1.0 + math.exp(-d))             # prob of the other class
        H_ref = -(q * math.log(q) + (1 - q) * math.log(1 - q))
        lp, H, _ = O.logprobs_entropy(z[None, :], [y], None, tau)
        assert abs(lp[0] - lp_ref) < 1e-12
        assert abs(H[0] - H_ref) < 1e-12


def test_two_class_closed_form():
    pin_two_class()


def pin_brute_force():
    rng = np.random.default_rng(2)
    for V in (1, 2, 3, 5, 8, 16):
        T = 6
        z = rng.normal(0, 2.5, size=(T, V))
        if V > 2:
            z[1, :] = 1.5               # ties everywhere
            z[2, 0] = z[2, 1] = z.max() + 1  # two equal maxima
        for tau in (1.0, 0.7, 1.9, -1.0, 0.0):
            for y in range(V):
                targets = np.full(T, y)
                lp, H, _ = O.logprobs_entropy(z, targets, None, tau)
                for t in range(T):
                    lp_ref, H_ref = bf_row(z[t], y, tau)
                    assert abs(lp[t] - lp_ref) < 1e-12, (V, tau, y, t)
                    assert abs(H[t] - H_ref) < 1e-12, (V, tau, y, t)


def test_brute_force_small_vocab():
    pin_brute_force()


def test_temperature_literal_reading():
    """tau <= 0 or tau == 1: no scaling (the helper's own condition)."""
    rng = np.random.default_rng(3)
    z = rng.normal(0, 3, size=(4, 33))
    y = rng.integers(0, 33, size=4)
    base = O.logprobs_entropy(z, y, None, 1.0)
    for tau in (-1.0, 0.0, -0.5):
        other = O.logprobs_entropy(z, y, None, tau)
        for a, b in zip(base, other):
            assert np.array_equal(a, b)
    # scaling identity: tau=0.5 on z equals tau=1 on 2z
    a = O.logprobs_entropy(z, y, None, 0.5)
    b = O.logprobs_entropy(2.0 * z, y, None, 1.0)
    for x1, x2 in zip(a, b):
        assert np.allclose(x1, x2, atol=1e-12, rtol=0)


def test_invariants_random_rows():
    rng = np.random.default_rng(4)
    for V in (3, 100, 4099):
        z = rng.normal(0, 4, size=(16, V))
        y = rng.integers(0, V, size=16)
        lp, H, lse = O.logprobs_entropy(z, y, None, 0.7)
        assert np.all(lp <= 1e-15)
        assert np.all(H >= -1e-15) and np.all(H <= math.log(V) + 1e-12)
        # lse bounds: max <= lse <= max + log V
        zt = z / 0.7
        assert np.all(lse >= zt.max(1) - 1e-12) and np.all(lse <= zt.max(1) + math.log(V) + 1e-12)


def test_one_hot_limit():
    V = 1000
    z = np.zeros((1, V))
    z[0, 17] = 100.0
    lp, H, _ = O.logprobs_entropy(z, [17], None, 1.0)
    eps = (V - 1) * math.exp(-100.0)
    assert abs(lp[0] + eps) < 1e-30
    assert 0.0 <= H[0] < 1e-38


def test_neg_inf_logits_add_nothing():
    z = np.array([[0.0, -np.inf, -np.inf, 0.0], [5.0, -np.inf, -np.inf, -np.inf]])
    lp, H, _ = O.logprobs_entropy(z, [0, 0], None, 0.7)
    assert abs(lp[0] + math.log(2)) < 1e-15 and abs(H[0] - math.log(2)) < 1e-15
    assert lp[1] == 0.0 and H[1] == 0.0


def test_unscored_rows_are_zero_and_targets_unread():
    rng = np.random.default_rng(5)
    z = rng.normal(size=(5, 9))
    targets = np.array([3, -100, 8, 10**9, 0])
    mask = np.array([1, 0, 1, 0, 1], dtype=np.uint8)
    lp, H, lse = O.logprobs_entropy(z, targets, mask, 0.7)
    assert lp[1] == 0 and H[1] == 0 and lp[3] == 0 and H[3] == 0 and lse[1] == 0
    assert np.all(np.isfinite(lp))


def test_out_of_range_target_poisons_logprob_only():
    z = np.zeros((2, 4))
    lp, H, _ = O.logprobs_entropy(z, [4, -1], None, 1.0)
    assert np.all(np.isnan(lp))
    assert np.allclose(H, math.log(4))


def test_empty_input():
    lp, H, lse = O.logprobs_entropy(np.zeros((0, 8)), np.zeros(0, dtype=np.int64), None, 0.7)
    assert lp.shape == (0,) and H.shape == (0,)
    assert O.chunk_plan(0, 4) == []


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def test_chunk_plan_page_example():
    """The page's worked example: 5 rows, chunk size 2 -> chunks of 2, 2, 1 rows."""
    lines = _read_golden("chunk_plan_5x8_c2.txt")
    T, V, c = (int(x) for x in lines[0].split())
    want = [int(x) for x in lines[1].split()]
    assert [n for _, n in O.chunk_plan(T, c)] == want
    # every row in exactly one chunk, in order
    plan = O.chunk_plan(T, c)
    assert [s for s, _ in plan] == [0, 2, 4]


def test_chunk_plan_reading():
    assert [n for _, n in O.chunk_plan(9, 4)] == [4, 4, 1]
    assert O.chunk_plan(7, 0) == [(0, 7)] and O.chunk_plan(7, -1) == [(0, 7)]
    assert O.chunk_plan(7, 100) == [(0, 7)]
    assert [n for _, n in O.chunk_plan(8192, 4096)] == [4096, 4096]


def test_chunking_does_not_change_rows():
    rng = np.random.default_rng(6)
    z = rng.normal(0, 3, size=(11, 257))
    y = rng.integers(0, 257, size=11)
    full = O.logprobs_entropy(z, y, None, 0.7)
    for c in (1, 3, 4, 11, 20):
        parts = [O.logprobs_entropy(z[s:s + n], y[s:s + n], None, 0.7) for s, n in O.chunk_plan(11, c)]
        for k in range(3):
            assert np.array_equal(np.concatenate([p[k] for p in parts]), full[k])


# ---------------------------------------------------------------------------
# pins: widening and rounding of inputs
# ---------------------------------------------------------------------------

def test_widen_known_bits():
    bf = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x4049], dtype=np.uint16)
    w = O.widen_bf16(bf)
    assert w[0] == 1.0 and w[1] == -2.0 and w[2] == np.inf and w[3] == -np.inf
    assert w[4] == 2.0 ** -133  # smallest bf16 subnormal
    assert w[5] == 3.140625
    hf = np.array([0x3C00, 0x7BFF, 0xFC00, 0x0001], dtype=np.uint16)
    w = O.widen_fp16(hf)
    assert w[0] == 1.0 and w[1] == 65504.0 and w[2] == -np.inf and w[3] == 2.0 ** -24


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5], dtype=np.float32)
    b = synth.f32_to_bf16_bits(x)
    assert list(O.widen_bf16(b)) == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5]


def test_generators_deterministic():
    a = synth.LogitsInput(T=64, V=300, run_lo=8, run_hi=20, chunk_rows=16).build().arrays
    b = synth.LogitsInput(T=64, V=300, run_lo=8, run_hi=20, chunk_rows=16).build().arrays
    for k in a:
        assert np.array_equal(a[k], b[k])
    frac = a["mask"].mean()
    assert 0.5 < frac < 0.95
    assert a["spike_rows"].sum() == round(0.3 * 64)


# ---------------------------------------------------------------------------
# pins: fused LM head forward and backward
# ---------------------------------------------------------------------------

def pin_lm_head_brute_force():
    rng = np.random.default_rng(7)
    T, h, V = 5, 3, 7
    Hm = rng.normal(size=(T, h))
    Wm = rng.normal(size=(V, h))
    y = rng.integers(0, V, size=T)
    mask = np.array([1, 1, 0, 1, 1])
    Z = bf_matmul_T(Hm.tolist(), Wm.tolist())
    for tau in (1.0, 0.7):
        lp, H, _ = O.lm_head_logprobs_entropy(Hm, Wm, y, mask, tau)
        for t in range(T):
            if not mask[t]:
                assert lp[t] == 0 and H[t] == 0
                continue
            lp_ref, H_ref = bf_row(Z[t], int(y[t]), tau)
            assert abs(lp[t] - lp_ref) < 1e-12 and abs(H[t] - H_ref) < 1e-12


def test_lm_head_brute_force():
    pin_lm_head_brute_force()


def test_lm_head_matches_logits_path_on_tiny_config():
    cfg = synth.tiny_lm_head()
    A = cfg.arrays
    Hd = O.widen_bf16(A["hidden"])
    Wd = O.widen_bf16(A["weight"])
    lp, H, lse = O.lm_head_logprobs_entropy(Hd, Wd, A["targets"], A["mask"], cfg.temperature)
    Z = bf_matmul_T(Hd[:2].tolist(), Wd.tolist())
    for t in range(2):
        lp_ref, H_ref = bf_row(Z[t], int(A["targets"][t]), cfg.temperature)
        assert abs(lp[t] - lp_ref) < 1e-11 and abs(H[t] - H_ref) < 1e-11


def pin_backward_finite_differences(tau=0.7, seed=8):
    rng = np.random.default_rng(seed)
    T, h, V = 4, 5, 6
    Hm = rng.normal(size=(T, h))
    Wm = rng.normal(0, 0.7, size=(V, h))
    y = rng.integers(0, V, size=T)
    mask = np.array([1, 0, 1, 1])
    g_lp = rng.normal(size=T)
    g_H = rng.normal(0, 0.5, size=T)
    dH, dW = O.lm_head_backward(Hm, Wm, y, mask, tau, g_lp, g_H)
    eps = 1e-5

    def L(Hx, Wx):
        return O.lm_head_loss(Hx, Wx, y, mask, tau, g_lp, g_H)

    for t in range(T):
        for k in range(h):
            Hp, Hn = Hm.copy(), Hm.copy()
            Hp[t, k] += eps
            Hn[t, k] -= eps
            fd = (L(Hp, Wm) - L(Hn, Wm)) / (2 * eps)
            assert abs(fd - dH[t, k]) <= 1e-6 * max(1.0, abs(fd)), ("dH", t, k, fd, dH[t, k])
    for j in range(V):
        for k in range(h):
            Wp, Wn = Wm.copy(), Wm.copy()
            Wp[j, k] += eps
            Wn[j, k] -= eps
            fd = (L(Hm, Wp) - L(Hm, Wn)) / (2 * eps)
            assert abs(fd - dW[j, k]) <= 1e-6 * max(1.0, abs(fd)), ("dW", j, k, fd, dW[j, k])


@pytest.mark.parametrize("tau", [1.0, 0.7, 1.6])
def test_backward_finite_differences(tau):
    pin_backward_finite_differences(tau)


def test_backward_invariants():
    rng = np.random.default_rng(9)
    T, h, V = 6, 8, 13
    Hm = rng.normal(size=(T, h))
    Wm = rng.normal(size=(V, h))
    y = rng.integers(0, V, size=T)
    mask = np.array([1, 1, 0, 1, 0, 1])
    g_lp, g_H = rng.normal(size=T), rng.normal(size=T)
    rows, dZ = O.lm_head_logit_grad(Hm, Wm, y, mask, 0.7, g_lp, g_H)
    assert list(rows) == [0, 1, 3, 5]
    assert np.allclose(dZ.sum(axis=1), 0.0, atol=1e-13)
    dH, dW = O.lm_head_backward(Hm, Wm, y, mask, 0.7, g_lp, g_H)
    assert np.all(dH[[2, 4]] == 0)
    # no scored rows: both gradients vanish
    dH0, dW0 = O.lm_head_backward(Hm, Wm, y, np.zeros(T), 0.7, g_lp, g_H)
    assert not dH0.any() and not dW0.any()
    # g_H = 0, tau = 1: dZ_t = g_lp,t (onehot - softmax(z_t)), written out by hand
    rows, dZ = O.lm_head_logit_grad(Hm, Wm, y, None, 1.0, g_lp, None)
    Z = bf_matmul_T(Hm.tolist(), Wm.tolist())
    for t in range(T):
        e = [math.exp(v) for v in Z[t]]
        S = math.fsum(e)
        for j in range(V):
            want = g_lp[t] * ((1.0 if j == y[t] else 0.0) - e[j] / S)
            assert abs(dZ[t, j] - want) < 1e-12


# ---------------------------------------------------------------------------
# pins: KL and prob diff
# ---------------------------------------------------------------------------

def test_kl_self_is_exactly_zero():
    rng = np.random.default_rng(10)
    u = rng.normal(0, 4, size=(8, 129))
    assert np.all(O.kl_full_vocab(u, u) == 0.0)


def pin_kl_two_class():
    rng = np.random.default_rng(11)
    for _ in range(40):
        u = rng.normal(0, 2, size=2)
        v = rng.normal(0, 2, size=2)
        q = 1 / (1 + math.exp(u[0] - u[1]))   # student prob of class 1
        p = 1 / (1 + math.exp(v[0] - v[1]))   # teacher prob of class 1
        want = p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
        got = O.kl_full_vocab(u[None], v[None])[0]
        assert abs(got - want) < 1e-12


def test_kl_two_class_bernoulli():
    pin_kl_two_class()


def pin_kl_brute_force():
    rng = np.random.default_rng(12)
    for V in (1, 2, 5, 16):
        u = rng.normal(0, 3, size=(5, V))
        v = u + rng.normal(0, 0.5, size=(5, V))
        got = O.kl_full_vocab(u, v)
        for t in range(5):
            assert abs(got[t] - bf_kl(u[t], v[t])) < 1e-12


def test_kl_brute_force():
    pin_kl_brute_force()


def test_kl_invariants():
    rng = np.random.default_rng(13)
    u = rng.normal(0, 4, size=(8, 1000))
    v = u + rng.normal(0, 0.5, size=u.shape)
    kl = O.kl_full_vocab(u, v)
    assert np.all(kl >= 0)
    # shifting a row by a constant leaves its distribution unchanged
    assert np.allclose(O.kl_full_vocab(u + 3.0, u), 0.0, atol=1e-12)


def test_prob_diff_page_cases():
    a = np.log(np.array([0.5, 0.25, 1.0, 0.125]))
    b = np.log(np.array([0.25, 0.25, 0.5, 0.5]))
    d = O.prob_diff(a, b, None)
    assert np.allclose(d, [0.25, 0.0, 0.5, 0.375], atol=1e-15, rtol=0)
    # all-False mask -> all-zero diff (msprobe edge-case table)
    assert np.all(O.prob_diff(a, b, np.zeros(4)) == 0)
    m = np.array([1, 0, 1, 0])
    assert np.allclose(O.prob_diff(a, b, m), [0.25, 0, 0.5, 0], atol=1e-15, rtol=0)
    assert np.all(O.prob_diff(a, a, None) == 0)


def test_kl_and_prob_diff_bundle():
    rng = np.random.default_rng(14)
    u = rng.normal(0, 4, size=(6, 50))
    v = u + rng.normal(0, 0.5, size=u.shape)
    y = rng.integers(0, 50, size=6)
    m = np.array([1, 0, 1, 1, 0, 1])
    kl, lpu, lpv, d = O.kl_and_prob_diff(u, v, y, m)
    for t in range(6):
        lpu_ref, _ = bf_row(u[t], int(y[t]), 1.0)
        lpv_ref, _ = bf_row(v[t], int(y[t]), 1.0)
        assert abs(lpu[t] - lpu_ref) < 1e-12 and abs(lpv[t] - lpv_ref) < 1e-12
        want = abs(math.exp(lpu_ref) - math.exp(lpv_ref)) if m[t] else 0.0
        assert abs(d[t] - want) < 1e-12


# ---------------------------------------------------------------------------
# negative controls: the pins are sensitive to the failure modes the pages name
# ---------------------------------------------------------------------------

def test_negative_control_temperature_in_model_precision():
    """Dividing by the temperature in bf16 (before the upcast) is measurably
    wrong on logits-input-like rows, so a kernel that matches the oracle to
    1e-5 cannot be doing it."""
    cfg = synth.LogitsInput(T=32, V=151936).build()
    A = cfg.arrays
    z = O.widen_bf16(A["logits"])
    lp, H, _ = O.logprobs_entropy(z, A["targets"], None, 0.7)
    z_bf16_div = O.widen_bf16(synth.f32_to_bf16_bits((z / 0.7).astype(np.float32)))
    lp2, H2, _ = O.logprobs_entropy(z_bf16_div, A["targets"], None, 1.0)
    assert max(np.abs(lp - lp2).max(), np.abs(H - H2).max()) > 1e-3


def test_negative_control_fp16_accumulation_overflows():
    cfg = synth.KLPair(T=4, V=129280).build()
    u = cfg.arrays["student"].view(np.float16)
    with np.errstate(over="ignore"):
        s16 = np.exp(u[0]).sum(dtype=np.float16)
        q16 = (u[0] * u[0]).sum(dtype=np.float16)
    assert np.isinf(s16) and np.isinf(q16)
    kl = O.kl_full_vocab(O.widen_fp16(cfg.arrays["student"]), O.widen_fp16(cfg.arrays["teacher"]))
    assert np.all(np.isfinite(kl))


# ---------------------------------------------------------------------------
# mutation tests: plant a mistake in the oracle, on the CPU; a pin must fail
# ---------------------------------------------------------------------------

def _must_fail(pin):
    with pytest.raises(AssertionError):
        pin()


def test_mutation_entropy_sign(monkeypatch):
    orig = O.shannon_entropy
    monkeypatch.setattr(O, "shannon_entropy", lambda lp: -orig(lp))
    _must_fail(pin_uniform)


def test_mutation_temperature_multiplied(monkeypatch):
    monkeypatch.setattr(O, "tempered", lambda z, t: np.asarray(z, float) * t if O.temperature_applies(t)
                        else np.asarray(z, float).copy())
    _must_fail(pin_two_class)


def test_mutation_dropped_max_shift_term(monkeypatch):
    def bad(zt):
        zt = np.atleast_2d(zt)
        return np.log(np.exp(zt - zt.max(1, keepdims=True)).sum(1))   # forgot + max
    monkeypatch.setattr(O, "log_normaliser", bad)
    _must_fail(pin_brute_force)


def test_mutation_wrong_vocab_index(monkeypatch):
    monkeypatch.setattr(O, "lm_head_logits", lambda Hd, W, vocab_block=0: (np.asarray(W, float) @ np.asarray(Hd, float).T).T[:, ::-1])
    _must_fail(pin_lm_head_brute_force)


def test_mutation_backward_drops_entropy_term(monkeypatch):
    orig = O.lm_head_logit_grad
    monkeypatch.setattr(O, "lm_head_logit_grad",
                        lambda Hm, Wm, y, m, tau, g_lp, g_H: orig(Hm, Wm, y, m, tau, g_lp, None))
    _must_fail(pin_backward_finite_differences)


def test_mutation_backward_missing_temperature(monkeypatch):
    orig = O.lm_head_logit_grad
    def bad(Hm, Wm, y, m, tau, g_lp, g_H):
        rows, dZ = orig(Hm, Wm, y, m, tau, g_lp, g_H)
        return rows, dZ * tau
    monkeypatch.setattr(O, "lm_head_logit_grad", bad)
    _must_fail(pin_backward_finite_differences)


def test_mutation_kl_direction(monkeypatch):
    orig = O.kl_full_vocab
    monkeypatch.setattr(O, "kl_full_vocab", lambda u, v: orig(v, u))
    _must_fail(pin_kl_two_class)


# ---------------------------------------------------------------------------
# pins: prob-diff aggregates and K targets per row
# ---------------------------------------------------------------------------

def test_prob_diff_stats_hand_values():
    pa = np.array([0.5, 0.25, 1.0, 0.125, 0.75])
    pb = np.array([0.25, 0.25, 0.5, 0.5, 0.75])
    m = np.array([1, 1, 1, 0, 1])
    n, mx, mean, std, r = O.prob_diff_stats(np.log(pa), np.log(pb), m)
    d = [0.25, 0.0, 0.5, 0.0]
    mu = sum(d) / 4
    assert n == 4 and abs(mx - 0.5) < 1e-15 and abs(mean - mu) < 1e-15
    assert abs(std - math.sqrt(sum((x - mu) ** 2 for x in d) / 4)) < 1e-15
    xa, xb = [0.5, 0.25, 1.0, 0.75], [0.25, 0.25, 0.5, 0.75]
    ma, mb = sum(xa) / 4, sum(xb) / 4
    cov = sum((u - ma) * (v - mb) for u, v in zip(xa, xb))
    va = sum((u - ma) ** 2 for u in xa)
    vb = sum((v - mb) ** 2 for v in xb)
    assert abs(r - cov / math.sqrt(va * vb)) < 1e-14


def test_prob_diff_stats_special_cases():
    rng = np.random.default_rng(30)
    p = rng.uniform(0.01, 0.5, size=100)
    # a linear relation has correlation exactly 1 (up to rounding); identical series give zero diff
    n, mx, mean, std, r = O.prob_diff_stats(np.log(p), np.log(0.5 * p + 0.1), None)
    assert n == 100 and abs(r - 1.0) < 1e-12
    n, mx, mean, std, r = O.prob_diff_stats(np.log(p), np.log(p), None)
    assert mx == 0 and mean == 0 and std == 0 and abs(r - 1.0) < 1e-12
    # all-False mask: nothing to aggregate
    n, mx, mean, std, r = O.prob_diff_stats(np.log(p), np.log(p), np.zeros(100))
    assert n == 0 and mx == 0 and mean == 0 and std == 0 and math.isnan(r)
    # one position, or a constant series: no spread, so no correlation
    n, mx, mean, std, r = O.prob_diff_stats(np.log([0.5]), np.log([0.25]), None)
    assert n == 1 and abs(mx - 0.25) < 1e-15 and abs(mean - 0.25) < 1e-15 and std == 0 and math.isnan(r)
    n, mx, mean, std, r = O.prob_diff_stats(np.log(np.full(5, 0.3)), np.log(p[:5]), None)
    assert n == 5 and math.isnan(r)


def test_k_targets_match_single_target_calls():
    rng = np.random.default_rng(31)
    z = rng.normal(0, 3, size=(7, 41))
    yk = rng.integers(0, 41, size=(7, 5))
    m = np.array([1, 1, 0, 1, 1, 0, 1])
    lpk, Hk, lsek = O.logprobs_entropy_k(z, yk, m, 0.7)
    for k in range(5):
        for t in range(7):
            if m[t]:
                lp_ref, H_ref = bf_row(z[t], int(yk[t, k]), 0.7)
                assert abs(lpk[t, k] - lp_ref) < 1e-12 and abs(Hk[t] - H_ref) < 1e-12
            else:
                assert lpk[t, k] == 0 and Hk[t] == 0


def test_k_target_backward_finite_differences():
    rng = np.random.default_rng(32)
    T, h, V, K = 3, 4, 5, 3
    Hm = rng.normal(size=(T, h))
    Wm = rng.normal(0, 0.7, size=(V, h))
    yk = rng.integers(0, V, size=(T, K))
    yk[0, 1] = yk[0, 0]  # a repeated target counts twice
    mask = np.array([1, 0, 1])
    g = rng.normal(size=(T, K))
    gH = rng.normal(0, 0.5, size=T)
    dH, dW = O.lm_head_backward_k(Hm, Wm, yk, mask, 0.7, g, gH)
    eps = 1e-5
    for (arr, grad) in ((Hm, dH), (Wm, dW)):
        for idx in np.ndindex(arr.shape):
            P, N = arr.copy(), arr.copy()
            P[idx] += eps
            N[idx] -= eps
            args_p = (P, Wm) if arr is Hm else (Hm, P)
            args_n = (N, Wm) if arr is Hm else (Hm, N)
            fd = (O.lm_head_loss_k(*args_p, yk, mask, 0.7, g, gH) - O.lm_head_loss_k(*args_n, yk, mask, 0.7, g, gH)) \
                / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, grad[idx])
    # K = 1 reduces to the single-target backward
    d1 = O.lm_head_backward_k(Hm, Wm, yk[:, :1], mask, 0.7, g[:, :1], gH)
    d0 = O.lm_head_backward(Hm, Wm, yk[:, 0], mask, 0.7, g[:, 0], gH)
    assert np.allclose(d1[0], d0[0], atol=1e-14) and np.allclose(d1[1], d0[1], atol=1e-14)


# ---------------------------------------------------------------------------
# pins: KL rebuilt through each model's output head
# ---------------------------------------------------------------------------

def _kl_heads(seed, T=4, hs=3, ht=5, V=6):
    rng = np.random.default_rng(seed)
    Hs = rng.normal(size=(T, hs))
    Ws = rng.normal(0, 0.8, size=(V, hs))
    Ht = rng.normal(size=(T, ht))
    Wt = rng.normal(0, 0.8, size=(V, ht))
    return Hs, Ws, Ht, Wt


def pin_lm_head_kl_brute_force():
    Hs, Ws, Ht, Wt = _kl_heads(40)
    T, V = Hs.shape[0], Ws.shape[0]
    y = np.array([2, 0, 5, 3])
    mask = np.array([1, 1, 0, 1])
    dmask = np.array([1, 0, 1, 1])
    kl, lpu, lpv, diff, lseu, lsev = O.lm_head_kl(Hs, Ws, Ht, Wt, mask, y, dmask)
    U = bf_matmul_T(Hs.tolist(), Ws.tolist())
    Vt = bf_matmul_T(Ht.tolist(), Wt.tolist())
    for t in range(T):
        if not mask[t]:
            assert kl[t] == lpu[t] == lpv[t] == diff[t] == lseu[t] == lsev[t] == 0
            continue
        assert abs(kl[t] - bf_kl(U[t], Vt[t])) < 1e-12
        a, _ = bf_row(U[t], int(y[t]), 1.0)
        b, _ = bf_row(Vt[t], int(y[t]), 1.0)
        assert abs(lpu[t] - a) < 1e-12 and abs(lpv[t] - b) < 1e-12
        want = abs(math.exp(a) - math.exp(b)) if dmask[t] else 0.0
        assert abs(diff[t] - want) < 1e-12
        assert abs(lseu[t] - math.log(math.fsum(math.exp(x) for x in U[t]))) < 1e-12
        assert abs(lsev[t] - math.log(math.fsum(math.exp(x) for x in Vt[t]))) < 1e-12


def test_lm_head_kl_brute_force():
    pin_lm_head_kl_brute_force()


def test_lm_head_kl_same_model_is_zero():
    Hs, Ws, _, _ = _kl_heads(41)
    kl = O.lm_head_kl(Hs, Ws, Hs, Ws, None, None, None)[0]
    assert np.all(kl == 0.0)
    dH, dW = O.lm_head_kl_backward(Hs, Ws, Hs, Ws, None, np.ones(Hs.shape[0]))
    assert not dH.any() and not dW.any()


def pin_lm_head_kl_backward_finite_differences():
    Hs, Ws, Ht, Wt = _kl_heads(42, T=3, hs=4, ht=2, V=5)
    mask = np.array([1, 0, 1])
    g = np.array([0.7, -1.3, 1.9])
    dH, dW = O.lm_head_kl_backward(Hs, Ws, Ht, Wt, mask, g)
    eps = 1e-5
    for arr, grad in ((Hs, dH), (Ws, dW)):
        for idx in np.ndindex(arr.shape):
            P, N = arr.copy(), arr.copy()
            P[idx] += eps
            N[idx] -= eps
            ap = (P, Ws) if arr is Hs else (Hs, P)
            an = (N, Ws) if arr is Hs else (Hs, N)
            fd = (O.lm_head_kl_loss(*ap, Ht, Wt, mask, g) - O.lm_head_kl_loss(*an, Ht, Wt, mask, g)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, grad[idx])


def test_lm_head_kl_backward_finite_differences():
    pin_lm_head_kl_backward_finite_differences()


def test_lm_head_kl_backward_vocab_sum_is_zero():
    # each row of dL/du sums to 0 (sum p_u - sum p_v), so dW summed over the vocab vanishes
    Hs, Ws, Ht, Wt = _kl_heads(43, T=6, hs=8, ht=8, V=40)
    _, dW = O.lm_head_kl_backward(Hs, Ws, Ht, Wt, None, np.linspace(-1, 2, 6))
    assert np.abs(dW.sum(axis=0)).max() < 1e-13


def test_mutation_lm_head_kl_models_swapped(monkeypatch):
    orig = O.lm_head_kl
    monkeypatch.setattr(O, "lm_head_kl", lambda hs, ws, ht, wt, m, y, d: orig(ht, wt, hs, ws, m, y, d))
    _must_fail(pin_lm_head_kl_brute_force)


def test_mutation_lm_head_kl_gradient_sign(monkeypatch):
    orig = O.lm_head_kl_backward
    def bad(*a):
        dH, dW = orig(*a)
        return -dH, -dW
    monkeypatch.setattr(O, "lm_head_kl_backward", bad)
    _must_fail(pin_lm_head_kl_backward_finite_differences)
