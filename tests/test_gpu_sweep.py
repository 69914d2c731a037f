"""Seeded sweep of random shapes through the fused LM head (forward and
recompute backward, one or several targets per row), the KL through both
heads (forward and student backward) and the logits-input rows, each
compared with the fp64 oracle.  The shapes mix hidden widths on
both tile paths (multiples of 64 take the direct-to-LDS tiles, the others the
generic ones), vocabularies from 1 to a few thousand (ragged last vocab
blocks), tile sizes below, inside and beyond the row count, all-, some- and
no-scored masks, and temperatures on both sides of 1.  Tolerances as in the
fixed-shape tests: abs 2e-3 on log-prob / entropy / lse of the fused head,
gradients relative Frobenius and max|diff| / max|ref| <= 1e-2, abs 1e-5 on
the logits-input rows."""
import numpy as np
import pytest

import synth
from oracle import lp_oracle as O
from tests.helpers import grad_errors, host, max_abs_err, to_dev, to_dev_bits

pytestmark = pytest.mark.gpu
TOL_FWD = 2e-3
TOL_GRAD = 1e-2
TOL_ROWS = 1e-5


def _cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        h = int(rng.choice([8, 24, 40, 64, 96, 128, 136, 192, 256]))
        V = int(rng.choice([1, 2, 7, 255, 256, 257, 700, 1031, 2049, 2200]))
        T = int(rng.integers(1, 521))
        tile = int(rng.choice([1, 5, 16, 64, 160, 256, 321, 4096]))
        tau = float(rng.choice([0.6, 1.0, 1.37]))
        scored = float(rng.choice([0.0, 0.35, 0.35, 0.35, 1.0, 1.0]))
        K = int(rng.choice([1, 1, 2, 3]))
        out.append((i, T, h, V, tile, tau, scored, K))
    return out


CASES = _cases(20261202, 64)


def _lp():
    import entropy_chunked_row_amd as lp
    return lp


@pytest.mark.parametrize("case", CASES, ids=lambda c: "i%d_T%d_h%d_V%d_tile%d_tau%g_s%g_K%d" % c)
def test_sweep_fused_head_forward_backward(case):
    i, T, h, V, tile, tau, scored, K = case
    rng = np.random.default_rng(1000 + i)
    hid = synth.f32_to_bf16_bits(rng.normal(0, 1, size=(T, h)).astype(np.float32))
    W = synth.f32_to_bf16_bits(rng.normal(0, 0.08, size=(V, h)).astype(np.float32))
    y = rng.integers(0, V, size=(T, K)).astype(np.int64)
    m = (rng.random(T) < scored).astype(np.uint8)
    g_lp = rng.normal(0, 1, size=(T, K)).astype(np.float32)
    g_H = rng.normal(0, 0.1, size=T).astype(np.float32)
    lp = _lp()
    hd, Wd, md = to_dev_bits(hid, "bf16"), to_dev_bits(W, "bf16"), to_dev(m)
    Hw, Ww = O.widen_bf16(hid), O.widen_bf16(W)
    if K == 1:
        lpv, H, lse = lp.lp_lm_head_logprobs_entropy(hd, Wd, to_dev(y[:, 0]), md, tau, tile)
        dH, dW = lp.lp_lm_head_logprobs_entropy_backward(hd, Wd, to_dev(y[:, 0]), md, tau, tile, lse, H,
                                                         to_dev(g_lp[:, 0]), to_dev(g_H))
        lp_o, H_o, lse_o = O.lm_head_logprobs_entropy(Hw, Ww, y[:, 0], m, tau)
        dH_o, dW_o = O.lm_head_backward(Hw, Ww, y[:, 0], m, tau, g_lp[:, 0], g_H)
        got_lp = host(lpv)
    else:
        lpv, H, lse = lp.lp_lm_head_logprobs_entropy_k(hd, Wd, to_dev(y), md, tau, tile)
        dH, dW = lp.lp_lm_head_logprobs_entropy_backward_k(hd, Wd, to_dev(y), md, tau, tile, lse, H, to_dev(g_lp),
                                                           to_dev(g_H))
        lp_o, H_o, lse_o = O.lm_head_logprobs_entropy_k(Hw, Ww, y, m, tau)
        dH_o, dW_o = O.lm_head_backward_k(Hw, Ww, y, m, tau, g_lp, g_H)
        got_lp = host(lpv)
    assert max_abs_err(got_lp, lp_o) <= TOL_FWD
    assert max_abs_err(host(H), H_o) <= TOL_FWD
    assert max_abs_err(host(lse), lse_o) <= TOL_FWD
    assert not got_lp[m == 0].any() and not host(H)[m == 0].any()
    for got, want in ((host(dH), dH_o), (host(dW), dW_o)):
        if not np.abs(want).max(initial=0.0) > 0:
            # an exactly-zero gradient (no scored rows, or V = 1 where p = 1 and the target terms cancel):
            # the fp32 kernels leave rounding residue of the cancelling terms, bounded by fp32 epsilon times
            # the size of those terms summed over the scored rows
            keep = m == 1
            scale = (np.abs(g_lp[keep]).sum() + np.abs(g_H[keep]).sum()) / tau * max(1.0, np.abs(Hw).max(),
                                                                                     np.abs(Ww).max())
            assert np.abs(got).max(initial=0.0) <= 1e-6 * scale + 1e-12, (np.abs(got).max(), scale)
            continue
        fro, mad = grad_errors(got, want)
        assert fro <= TOL_GRAD and mad <= TOL_GRAD, (fro, mad)


ROW_CASES = _cases(71, 24)


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: "i%d_T%d_V%d_tau%g_s%g_K%d" % (c[0], c[1], c[3], c[5], c[6],
                                                                                          c[7]))
def test_sweep_logits_rows(case):
    i, T, _, V, tile, tau, scored, K = case
    rng = np.random.default_rng(2000 + i)
    logits = synth.f32_to_bf16_bits(rng.normal(0, 2.0, size=(T, V)).astype(np.float32))
    y = rng.integers(0, V, size=(T, K)).astype(np.int64)
    m = (rng.random(T) < scored).astype(np.uint8)
    chunk = int(rng.choice([-1, 1, 7, 64, 4096]))
    lp = _lp()
    x = to_dev_bits(logits, "bf16")
    if K == 1:
        got_lp, got_H = lp.lp_logprobs_entropy(x, to_dev(y[:, 0]), to_dev(m), tau, chunk)
        want_lp, want_H, _ = O.logprobs_entropy(O.widen_bf16(logits), y[:, 0], m, tau)
    else:
        got_lp, got_H = lp.lp_logprobs_entropy_k(x, to_dev(y), to_dev(m), tau, chunk)
        want_lp, want_H, _ = O.logprobs_entropy_k(O.widen_bf16(logits), y, m, tau)
    assert max_abs_err(host(got_lp), want_lp) <= TOL_ROWS
    assert max_abs_err(host(got_H), want_H) <= TOL_ROWS


KL_CASES = _cases(5151, 24)


@pytest.mark.parametrize("case", KL_CASES, ids=lambda c: "i%d_T%d_h%d_V%d_tile%d_s%g" % (c[0], c[1], c[2], c[3], c[4],
                                                                                        c[6]))
def test_sweep_kl_heads_forward_backward(case):
    i, T, hs, V, tile, _, scored, _ = case
    rng = np.random.default_rng(3000 + i)
    ht = int(rng.choice([8, 40, 64, 72, 128, 200, 256]))  # the teacher's width, independent of the student's
    bf = lambda shape, sigma: synth.f32_to_bf16_bits(rng.normal(0, sigma, size=shape).astype(np.float32))
    Hs, Ws, Ht, Wt = bf((T, hs), 1.0), bf((V, hs), 0.08), bf((T, ht), 1.0), bf((V, ht), 0.08)
    m = (rng.random(T) < scored).astype(np.uint8)
    y = rng.integers(0, V, size=T).astype(np.int64)
    dm = (rng.random(T) < 0.6).astype(np.uint8)
    g = rng.normal(0, 1, size=T).astype(np.float32)
    lp = _lp()
    heads = [to_dev_bits(a, "bf16") for a in (Hs, Ws, Ht, Wt)]
    wide = [O.widen_bf16(a) for a in (Hs, Ws, Ht, Wt)]
    got = [host(t) for t in lp.lp_lm_head_kl(*heads, to_dev(m), to_dev(y), to_dev(dm), tile)]
    want = O.lm_head_kl(*wide, m, y, dm)
    for name, a, b in zip(("kl", "lp_s", "lp_t", "diff", "lse_s", "lse_t"), got, want):
        assert max_abs_err(a, b) <= TOL_FWD, (name, max_abs_err(a, b))
        assert not a[m == 0].any(), name
    dH, dW = lp.lp_lm_head_kl_backward(*heads, to_dev(m), tile, to_dev(got[4]), to_dev(got[5]), to_dev(g))
    dH_o, dW_o = O.lm_head_kl_backward(*wide, m, g)
    for nm, a, b in (("dH", host(dH), dH_o), ("dW", host(dW), dW_o)):
        if not np.abs(b).max(initial=0.0) > 0:
            # no scored rows, or V = 1 (both heads put probability 1 on the one column: KL = 0 everywhere)
            assert np.abs(a).max(initial=0.0) <= 1e-6 * max(1.0, np.abs(g[m == 1]).sum()) * max(
                1.0, np.abs(wide[0]).max(), np.abs(wide[1]).max()), nm
            continue
        fro, mad = grad_errors(a, b)
        assert fro <= TOL_GRAD and mad <= TOL_GRAD, (nm, fro, mad)
