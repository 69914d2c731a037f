"""GPU parity of the widened rows: K targets per row (logits input and fused
LM head, forward and backward) and the prob-diff aggregates."""
import math

import numpy as np
import pytest

import synth
from oracle import lp_oracle as O
from tests.helpers import grad_errors, host, max_abs_err, to_dev, to_dev_bits

pytestmark = pytest.mark.gpu


def _lp():
    import entropy_chunked_row_amd as lp
    return lp


@pytest.mark.parametrize("V,K", [(7, 1), (1031, 3), (20011, 8), (151936, 64)])
def test_logprobs_entropy_k(V, K):
    rng = np.random.default_rng(V + K)
    T = 9 if V > 100000 else 33
    x = synth.f32_to_bf16_bits(rng.normal(0, 3, size=(T, V)).astype(np.float32))
    yk = rng.integers(0, V, size=(T, K)).astype(np.int64)
    yk[0, -1] = V  # out of range -> NaN for that entry only
    m = (rng.random(T) < 0.8).astype(np.uint8)
    m[0] = 1
    lp, H = _lp().lp_logprobs_entropy_k(to_dev_bits(x, "bf16"), to_dev(yk), to_dev(m), 0.7, 4)
    lp, H = host(lp), host(H)
    lp_o, H_o, _ = O.logprobs_entropy_k(O.widen_bf16(x), yk, m, 0.7)
    assert np.isnan(lp[0, -1]) and np.isnan(lp_o[0, -1])
    ok = ~np.isnan(lp_o)
    assert max_abs_err(lp[ok], lp_o[ok]) <= 1e-5 and max_abs_err(H, H_o) <= 1e-5
    assert not lp[m == 0].any()


def test_k1_matches_single_target_bitwise():
    rng = np.random.default_rng(3)
    x = synth.f32_to_bf16_bits(rng.normal(0, 3, size=(20, 5003)).astype(np.float32))
    y = rng.integers(0, 5003, size=20).astype(np.int64)
    a, ha = _lp().lp_logprobs_entropy(to_dev_bits(x, "bf16"), to_dev(y), None, 0.7)
    b, hb = _lp().lp_logprobs_entropy_k(to_dev_bits(x, "bf16"), to_dev(y[:, None]), None, 0.7)
    assert np.array_equal(host(a), host(b)[:, 0]) and np.array_equal(host(ha), host(hb))


@pytest.mark.parametrize("T,h,V,K,tile", [(40, 64, 1031, 4, 16), (300, 256, 5000, 16, 128),
                                            (45, 72, 777, 3, 16)])  # the last: generic tiles (h % 64 != 0)
def test_lm_head_k_forward_backward(T, h, V, K, tile):
    rng = np.random.default_rng(T + K)
    hid = synth.f32_to_bf16_bits(rng.normal(0, 1, size=(T, h)).astype(np.float32))
    W = synth.f32_to_bf16_bits(rng.normal(0, 0.05, size=(V, h)).astype(np.float32))
    yk = rng.integers(0, V, size=(T, K)).astype(np.int64)
    yk[:, 1] = yk[:, 0]  # repeated targets
    m = (rng.random(T) < 0.7).astype(np.uint8)
    g = rng.normal(0, 1, size=(T, K)).astype(np.float32)
    gH = rng.normal(0, 0.1, size=T).astype(np.float32)
    hd, Wd = to_dev_bits(hid, "bf16"), to_dev_bits(W, "bf16")
    lp, H, lse = _lp().lp_lm_head_logprobs_entropy_k(hd, Wd, to_dev(yk), to_dev(m), 0.7, tile)
    lp_o, H_o, lse_o = O.lm_head_logprobs_entropy_k(O.widen_bf16(hid), O.widen_bf16(W), yk, m, 0.7)
    assert max_abs_err(host(lp), lp_o) <= 2e-3 and max_abs_err(host(H), H_o) <= 2e-3
    dH, dW = _lp().lp_lm_head_logprobs_entropy_backward_k(hd, Wd, to_dev(yk), to_dev(m), 0.7, tile, lse, H,
                                                          to_dev(g), to_dev(gH))
    dH_o, dW_o = O.lm_head_backward_k(O.widen_bf16(hid), O.widen_bf16(W), yk, m, 0.7, g, gH)
    for got, want in ((host(dH), dH_o), (host(dW), dW_o)):
        fro, mad = grad_errors(got, want)
        assert fro <= 1e-2 and mad <= 1e-2, (fro, mad)


@pytest.mark.parametrize("n", [1, 1000, 3_000_001])
def test_prob_diff_stats(n):
    rng = np.random.default_rng(n)
    a = np.log(rng.uniform(1e-4, 1.0, size=n)).astype(np.float32)
    b = (a + rng.normal(0, 0.05, size=n)).astype(np.float32)
    b = np.minimum(b, 0.0).astype(np.float32)
    m = (rng.random(n) < 0.6).astype(np.uint8)
    m[0] = 1
    got = host(_lp().lp_prob_diff_stats(to_dev(a), to_dev(b), to_dev(m)))
    want = O.prob_diff_stats(a.astype(np.float64), b.astype(np.float64), m)
    assert got[0] == want[0]
    assert abs(got[1] - want[1]) <= 1e-12 and abs(got[2] - want[2]) <= 1e-12
    assert abs(got[3] - want[3]) <= 1e-9
    if n > 1:
        assert abs(got[4] - want[4]) <= 1e-9
    else:
        assert math.isnan(got[4]) and math.isnan(want[4])
    again = host(_lp().lp_prob_diff_stats(to_dev(a), to_dev(b), to_dev(m)))
    assert np.array_equal(got, again, equal_nan=True)


def test_prob_diff_stats_edge_cases():
    a = np.log(np.array([0.5, 0.25, 0.75], dtype=np.float32))
    got = host(_lp().lp_prob_diff_stats(to_dev(a), to_dev(a), to_dev(np.zeros(3, np.uint8))))
    assert got[0] == 0 and got[1] == 0 and got[2] == 0 and got[3] == 0 and math.isnan(got[4])
    got = host(_lp().lp_prob_diff_stats(to_dev(a), to_dev(a), None))
    assert got[0] == 3 and got[1] == 0 and got[2] == 0 and abs(got[4] - 1.0) < 1e-12
