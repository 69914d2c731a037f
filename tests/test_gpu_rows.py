"""GPU parity of the logits-input path, exact KL and prob diff against the
fp64 oracle.  Tolerances: abs 1e-5 on log-prob / entropy / KL / diff (the
logits-input bar; KL and diff take the same bar as a reading)."""
import math

import numpy as np
import pytest

import synth
from oracle import lp_oracle as O
from tests.helpers import oracle_by_row_blocks, host, max_abs_err, to_dev, to_dev_bits

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _lp():
    import entropy_chunked_row_amd as lp
    return lp


def _torch():
    import torch
    return torch


def _random_case(T, V, dtype, sigma, seed, scored=0.75):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, sigma, size=(T, V)).astype(np.float32)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x)
    elif dtype == "fp16":
        bits = synth.f32_to_fp16_bits(x)
    else:
        bits = x
    targets = rng.integers(0, V, size=T).astype(np.int64)
    mask = (rng.random(T) < scored).astype(np.uint8)
    return bits, targets, mask


def _widen(bits, dtype):
    return O.widen(bits, dtype)


def _dev_logits(bits, dtype):
    if dtype == "fp32":
        return to_dev(bits)
    return to_dev_bits(bits, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("V", [1, 2, 3, 7, 16, 1000, 1031, 4099, 20011])
@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_logprobs_entropy_small(dtype, V, tau):
    T = 37
    bits, targets, mask = _random_case(T, V, dtype, 3.0, seed=V * 7 + int(tau * 10))
    lp, H = _lp().lp_logprobs_entropy(_dev_logits(bits, dtype), to_dev(targets), to_dev(mask), tau, 5)
    lp_o, H_o, _ = O.logprobs_entropy(_widen(bits, dtype), targets, mask, tau)
    assert max_abs_err(host(lp), lp_o) <= TOL
    assert max_abs_err(host(H), H_o) <= TOL
    assert np.all(host(lp)[mask == 0] == 0) and np.all(host(H)[mask == 0] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_padded_and_misaligned_rows(dtype):
    """ld > V and a row start off the 16-byte grid exercise head/tail handling."""
    torch = _torch()
    T, V, ld = 9, 3001, 3011
    bits, targets, mask = _random_case(T, ld, dtype, 3.0, seed=11)
    full = _dev_logits(bits, dtype)
    view = full[:, 3:3 + V]  # starts 6 bytes into the row, ld = 3011
    lp, H = _lp().lp_logprobs_entropy(view, to_dev(targets % V), to_dev(mask), 0.7, 4)
    lp_o, H_o, _ = O.logprobs_entropy(_widen(bits, dtype)[:, 3:3 + V], targets % V, mask, 0.7)
    assert max_abs_err(host(lp), lp_o) <= TOL and max_abs_err(host(H), H_o) <= TOL
    del torch


def test_chunking_is_bitwise_invariant():
    T, V = 29, 5003
    bits, targets, mask = _random_case(T, V, "bf16", 3.0, seed=12)
    x = _dev_logits(bits, "bf16")
    y, m = to_dev(targets), to_dev(mask)
    ref = [host(t) for t in _lp().lp_logprobs_entropy(x, y, m, 0.7, -1)]
    for c in (0, 1, 3, 4, 28, 29, 100):
        got = [host(t) for t in _lp().lp_logprobs_entropy(x, y, m, 0.7, c)]
        assert all(np.array_equal(a, b) for a, b in zip(ref, got)), c


def test_temperature_literal_reading_and_repeatability():
    T, V = 8, 777
    bits, targets, _ = _random_case(T, V, "bf16", 3.0, seed=13)
    x, y = _dev_logits(bits, "bf16"), to_dev(targets)
    base = [host(t) for t in _lp().lp_logprobs_entropy(x, y, None, 1.0)]
    for tau in (-1.0, 0.0, -3.0):
        got = [host(t) for t in _lp().lp_logprobs_entropy(x, y, None, tau)]
        assert all(np.array_equal(a, b) for a, b in zip(base, got))
    again = [host(t) for t in _lp().lp_logprobs_entropy(x, y, None, 1.0)]
    assert all(np.array_equal(a, b) for a, b in zip(base, again))


def test_uniform_rows_closed_form():
    torch = _torch()
    V = 151936
    x = torch.full((3, V), 2.5, dtype=torch.bfloat16, device="cuda")
    lp, H = _lp().lp_logprobs_entropy(x, to_dev(np.array([0, 5, V - 1])), None, 0.7)
    assert np.allclose(host(lp), -math.log(V), atol=TOL, rtol=0)
    assert np.allclose(host(H), math.log(V), atol=TOL, rtol=0)


def test_special_values_and_targets():
    torch = _torch()
    x = np.zeros((4, 10), dtype=np.float32)
    x[0, 3:] = -np.inf            # 3 equal live entries
    x[1, :] = 5.0
    x[1, 9] = -np.inf
    x[2, 0] = 100.0               # one-hot limit
    bits = synth.f32_to_bf16_bits(x)
    targets = np.array([0, 9, 0, 10], dtype=np.int64)  # row 3: out of range
    lp, H = _lp().lp_logprobs_entropy(_dev_logits(bits, "bf16"), to_dev(targets), None, 1.0)
    lp, H = host(lp), host(H)
    assert abs(lp[0] + math.log(3)) <= TOL and abs(H[0] - math.log(3)) <= TOL
    assert lp[1] == -np.inf or lp[1] < -1e30 or np.isneginf(lp[1])
    assert abs(H[1] - math.log(9)) <= TOL
    assert abs(lp[2]) <= TOL and abs(H[2]) <= TOL
    assert np.isnan(lp[3]) and abs(H[3] - math.log(10)) <= TOL
    del torch


def test_empty_and_input_untouched():
    torch = _torch()
    lp = _lp()
    x = torch.zeros((0, 100), dtype=torch.bfloat16, device="cuda")
    a, b = lp.lp_logprobs_entropy(x, torch.zeros(0, dtype=torch.int64, device="cuda"), None, 0.7, 4)
    assert a.numel() == 0 and b.numel() == 0
    bits, targets, mask = _random_case(16, 999, "bf16", 3.0, seed=14)
    xd = _dev_logits(bits, "bf16")
    before = xd.clone()
    lp.lp_logprobs_entropy(xd, to_dev(targets), to_dev(mask), 0.7, 3)
    assert torch.equal(before.view(torch.int16), xd.view(torch.int16))


def test_invalid_arguments_launch_nothing():
    torch = _torch()
    lp = _lp()
    x = torch.zeros((4, 8), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(4, dtype=torch.int64, device="cuda")
    out = torch.full((4,), 7.0, device="cuda")
    with pytest.raises(lp.LPError):
        lp.lp_logprobs_entropy(x, y, None, float("nan"), logprob=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# ---------------------------------------------------------------------------
# full-size logits-input workload: 8192 x 151936 bf16, tau 0.7, chunk 4096
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def logits_full():
    cfg = synth.LogitsInput().build()
    A = cfg.arrays
    return cfg, A, _dev_logits(A["logits"], "bf16"), to_dev(A["targets"]), to_dev(A["mask"])


@pytest.mark.timeout(600)
def test_full_size_logits_every_scored_row(logits_full):
    """Every scored row of the full workload (about 6000 rows of 151936
    logits, two chunks of 4096) against the fp64 oracle, which runs over row
    blocks in a thread pool."""
    cfg, A, x, y, m = logits_full
    lp, H = _lp().lp_logprobs_entropy(x, y, m, cfg.temperature, cfg.chunk_rows)
    lp, H = host(lp), host(H)
    scored = np.nonzero(A["mask"])[0]

    def oracle(rows):
        return O.logprobs_entropy(O.widen_bf16(A["logits"][rows]), A["targets"][rows], None, cfg.temperature)[:2]

    lp_o, H_o = oracle_by_row_blocks(oracle, scored)
    assert max_abs_err(lp[scored], lp_o) <= TOL, max_abs_err(lp[scored], lp_o)
    assert max_abs_err(H[scored], H_o) <= TOL, max_abs_err(H[scored], H_o)
    spikes = A["spike_rows"][scored].astype(bool)
    assert spikes.sum() > 1000  # the +8 target spikes are among the rows compared
    assert np.all(lp[A["mask"] == 0] == 0) and np.all(H[A["mask"] == 0] == 0)
    assert np.all(lp[scored] <= 1e-6) and np.all(H[scored] >= -1e-6)
    assert np.all(H[scored] <= math.log(cfg.V) + 1e-5)


# ---------------------------------------------------------------------------
# KL + prob diff
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("V", [1, 2, 5, 16, 1000, 4097, 129280])
def test_kl_small(dtype, V):
    T = 6 if V > 5000 else 23
    rng = np.random.default_rng(V)
    u = rng.normal(0, 4, size=(T, V)).astype(np.float32)
    v = u + rng.normal(0, 0.5, size=u.shape).astype(np.float32)
    conv = synth.f32_to_fp16_bits if dtype == "fp16" else synth.f32_to_bf16_bits
    ub, vb = conv(u), conv(v)
    targets = rng.integers(0, V, size=T).astype(np.int64)
    dm = (rng.random(T) < 0.6).astype(np.uint8)
    kl, lpu, lpv, d = _lp().lp_kl_full_vocab(to_dev_bits(ub, dtype), to_dev_bits(vb, dtype), to_dev(targets),
                                             to_dev(dm))
    kl_o, lpu_o, lpv_o, d_o = O.kl_and_prob_diff(O.widen(ub, dtype), O.widen(vb, dtype), targets, dm)
    assert max_abs_err(host(kl), kl_o) <= TOL
    assert max_abs_err(host(lpu), lpu_o) <= TOL and max_abs_err(host(lpv), lpv_o) <= TOL
    assert max_abs_err(host(d), d_o) <= TOL
    assert np.all(host(d)[dm == 0] == 0)


@pytest.mark.parametrize("V", [3, 1000, 4099])
def test_kl_fp32_inputs(V):
    T = 17
    rng = np.random.default_rng(V + 1)
    u = rng.normal(0, 4, size=(T, V)).astype(np.float32)
    v = (u + rng.normal(0, 0.5, size=u.shape)).astype(np.float32)
    targets = rng.integers(0, V, size=T).astype(np.int64)
    kl, lpu, lpv, d = _lp().lp_kl_full_vocab(to_dev(u), to_dev(v), to_dev(targets), None)
    kl_o, lpu_o, lpv_o, d_o = O.kl_and_prob_diff(u.astype(np.float64), v.astype(np.float64), targets, None)
    assert max_abs_err(host(kl), kl_o) <= TOL
    assert max_abs_err(host(lpu), lpu_o) <= TOL and max_abs_err(host(d), d_o) <= TOL


def test_kl_self_exactly_zero_and_no_targets():
    rng = np.random.default_rng(3)
    ub = synth.f32_to_fp16_bits(rng.normal(0, 4, size=(5, 3333)).astype(np.float32))
    x = to_dev_bits(ub, "fp16")
    kl, a, b, c = _lp().lp_kl_full_vocab(x, x.clone())
    assert np.all(host(kl) == 0.0) and a is None and b is None and c is None


@pytest.fixture(scope="module")
def kl_full():
    cfg = synth.KLPair().build()
    A = cfg.arrays
    return cfg, A, to_dev_bits(A["student"], "fp16"), to_dev_bits(A["teacher"], "fp16"), \
        to_dev(A["targets"]), to_dev(A["diff_mask"])


@pytest.mark.timeout(900)
def test_kl_full_size_every_row(kl_full):
    """Every row of the full workload (16384 rows of 129280 fp16 logits per
    model) against the fp64 oracle: KL, both target log-probs and the masked
    prob diff."""
    cfg, A, u, v, y, dm = kl_full
    kl, lpu, lpv, d = (host(t) for t in _lp().lp_kl_full_vocab(u, v, y, dm))

    def oracle(rows):
        return O.kl_and_prob_diff(O.widen_fp16(A["student"][rows]), O.widen_fp16(A["teacher"][rows]),
                                  A["targets"][rows], A["diff_mask"][rows])

    kl_o, lpu_o, lpv_o, d_o = oracle_by_row_blocks(oracle, np.arange(cfg.T), block=64)
    assert max_abs_err(kl, kl_o) <= TOL, max_abs_err(kl, kl_o)
    assert max_abs_err(lpu, lpu_o) <= TOL and max_abs_err(lpv, lpv_o) <= TOL
    assert max_abs_err(d, d_o) <= TOL
    assert np.all(np.isfinite(kl)) and np.all(kl >= -1e-5)
    assert np.all(d[A["diff_mask"] == 0] == 0)


def test_prob_diff_elementwise():
    rng = np.random.default_rng(4)
    n = 100003
    a = -np.abs(rng.normal(0, 3, n)).astype(np.float32)
    b = -np.abs(rng.normal(0, 3, n)).astype(np.float32)
    m = (rng.random(n) < 0.6).astype(np.uint8)
    got = host(_lp().lp_prob_diff(to_dev(a), to_dev(b), to_dev(m)))
    assert max_abs_err(got, O.prob_diff(a.astype(np.float64), b.astype(np.float64), m)) <= 1e-6
    assert np.all(host(_lp().lp_prob_diff(to_dev(a), to_dev(b), to_dev(np.zeros(n, np.uint8)))) == 0)


@pytest.mark.timeout(600)
def test_logits_past_4_gib():
    """Maximum-size case for the logits path: bf16 logits [30000, 151936]
    (9.1 GB), scored rows on both sides of the 4 GiB byte offset, in chunks."""
    import torch
    T, V = 30000, 151936
    rng = np.random.default_rng(98)
    rows = np.array([0, 14130, 14136, 14137, 20000, T - 1])
    vals = synth.f32_to_bf16_bits(rng.normal(0, 3, size=(len(rows), V)).astype(np.float32))
    y = rng.integers(0, V, size=T).astype(np.int64)
    mask = np.zeros(T, dtype=np.uint8)
    mask[rows] = 1
    x = torch.zeros((T, V), dtype=torch.bfloat16, device="cuda")
    x[torch.as_tensor(rows).cuda()] = to_dev_bits(vals, "bf16")
    lp, H = _lp().lp_logprobs_entropy(x, to_dev(y), to_dev(mask), 0.7, 8192)
    lp_o, H_o = O.logprobs_entropy(O.widen_bf16(vals), y[rows], None, 0.7)[:2]
    lph, Hh = host(lp), host(H)
    assert max_abs_err(lph[rows], lp_o) <= TOL and max_abs_err(Hh[rows], H_o) <= TOL
    assert not lph[mask == 0].any() and not Hh[mask == 0].any()


@pytest.mark.parametrize("V", [1, 2, 5, 16])
@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_brute_force_adversarial_small_vocab(V, tau):
    """GPU against the pure-Python brute force (math.fsum softmax, no max
    shift) on adversarial rows: all equal, two equal maxima, a -inf entry,
    large magnitudes, and random rows; every target id of every row."""
    from tests.test_oracle_pins import bf_row
    rng = np.random.default_rng(V * 10 + int(tau * 10))
    rows = [np.zeros(V), rng.normal(0, 3, V), np.full(V, 7.5)]
    if V >= 2:
        r = rng.normal(0, 1, V)
        r[0] = r[V - 1] = r.max() + 2.0  # two equal maxima
        rows.append(r)
        r = rng.normal(0, 2, V)
        r[V // 2] = -np.inf
        rows.append(r)
        rows.append(rng.uniform(-40, 40, V))
    Z = np.array(rows, dtype=np.float32)
    n = Z.shape[0]
    for y_col in range(V):
        y = np.full(n, y_col, dtype=np.int64)
        lp, H = _lp().lp_logprobs_entropy(to_dev(Z), to_dev(y), None, tau)
        lp, H = host(lp), host(H)
        for t in range(n):
            if not np.isfinite(Z[t, y_col]):
                continue
            want_lp, want_H = bf_row([float(v) for v in Z[t]], y_col, tau)
            assert abs(lp[t] - want_lp) <= TOL * max(1.0, abs(want_lp)), (t, y_col, lp[t], want_lp)
            assert abs(H[t] - want_H) <= TOL, (t, H[t], want_H)


@pytest.mark.timeout(600)
def test_more_rows_than_one_launch():
    """Row counts past one launch's 2^22 workgroups: the logits kernel (one
    chunk of all rows) and the KL on given logits split their launches;
    every row, including both sides of each split, against the oracle."""
    T, V = (1 << 22) + 4099, 5
    rng = np.random.default_rng(2222)
    u = rng.normal(0, 3, size=(T, V)).astype(np.float32)
    v = u + rng.normal(0, 0.5, size=u.shape).astype(np.float32)
    ub, vb = synth.f32_to_bf16_bits(u), synth.f32_to_bf16_bits(v)
    targets = rng.integers(0, V, size=T).astype(np.int64)
    mask = (rng.random(T) < 0.75).astype(np.uint8)
    lp, H = _lp().lp_logprobs_entropy(to_dev_bits(ub, "bf16"), to_dev(targets), to_dev(mask), 0.7, 0)
    lp_o, H_o, _ = O.logprobs_entropy(O.widen_bf16(ub), targets, mask, 0.7)
    assert max_abs_err(host(lp), lp_o) <= TOL and max_abs_err(host(H), H_o) <= TOL
    kl, lpu, lpv, d = _lp().lp_kl_full_vocab(to_dev_bits(ub, "bf16"), to_dev_bits(vb, "bf16"), to_dev(targets),
                                             to_dev(mask))
    kl_o, lpu_o, lpv_o, d_o = O.kl_and_prob_diff(O.widen_bf16(ub), O.widen_bf16(vb), targets, mask)
    for g, w in ((kl, kl_o), (lpu, lpu_o), (lpv, lpv_o), (d, d_o)):
        assert max_abs_err(host(g), w) <= TOL
