"""GPU parity of the KL rebuilt through each model's output head (forward
and student backward) against the fp64 oracle."""
import numpy as np
import pytest

import synth
from oracle import lp_oracle as O
from tests.helpers import grad_errors, host, max_abs_err, to_dev, to_dev_bits

pytestmark = pytest.mark.gpu

# Fused class: the logits are fp32 MFMA sums, compared with exact fp64 ones.
TOL_FWD = 2e-3
TOL_GRAD = 1e-2


def _lp():
    import entropy_chunked_row_amd as lp
    return lp


def _bf16(rng, shape, sigma):
    return synth.f32_to_bf16_bits((rng.normal(0, sigma, size=shape)).astype(np.float32))


def _case(T, hs, ht, V, seed, scored=0.8):
    rng = np.random.default_rng(seed)
    A = dict(student_hidden=_bf16(rng, (T, hs), 1.0), student_weight=_bf16(rng, (V, hs), 0.08),
             teacher_hidden=_bf16(rng, (T, ht), 1.0), teacher_weight=_bf16(rng, (V, ht), 0.08))
    A["mask"] = (rng.random(T) < scored).astype(np.uint8)
    A["targets"] = rng.integers(0, V, size=T).astype(np.int64)
    A["diff_mask"] = (rng.random(T) < 0.6).astype(np.uint8)
    A["grad_kl"] = rng.normal(0, 1, size=T).astype(np.float32)
    return A


def _dev_heads(A):
    return [to_dev_bits(A[k], "bf16") for k in ("student_hidden", "student_weight", "teacher_hidden",
                                                 "teacher_weight")]


def _wide(A):
    return [O.widen_bf16(A[k]) for k in ("student_hidden", "student_weight", "teacher_hidden", "teacher_weight")]


@pytest.mark.parametrize("T,hs,ht,V,tile", [
    (50, 40, 72, 1031, 16),      # generic path (h % 64 != 0), ragged tiles and vocab block
    (300, 128, 256, 5000, 128),  # fast path, different widths, partial last vocab block
    (70, 64, 72, 999, 32),       # student width on the fast path, teacher width not
    (130, 64, 64, 512, 4096),    # fast path, one tile, vocab a multiple of the block
])
def test_kl_head_forward_backward(T, hs, ht, V, tile):
    A = _case(T, hs, ht, V, seed=T + hs + ht)
    A["targets"][np.nonzero(A["mask"])[0][0]] = V  # out of range: NaN lps for that row only
    heads = _dev_heads(A)
    m, y, dm = to_dev(A["mask"]), to_dev(A["targets"]), to_dev(A["diff_mask"])
    got = [host(t) for t in _lp().lp_lm_head_kl(*heads, m, y, dm, tile)]
    want = O.lm_head_kl(*_wide(A), A["mask"], A["targets"], A["diff_mask"])
    sc = A["mask"] != 0
    bad = A["targets"] >= V
    for name, g, w in zip(("kl", "lp_s", "lp_t", "diff", "lse_s", "lse_t"), got, want):
        assert not g[~sc].any(), name
        ok = sc & ~bad if name in ("lp_s", "lp_t", "diff") else sc
        assert max_abs_err(g[ok], w[ok]) <= TOL_FWD, (name, max_abs_err(g[ok], w[ok]))
    assert np.isnan(got[1][bad]).all() and np.isfinite(got[0][sc]).all()
    # rows do not depend on the tiling: bitwise equal with another tile size
    again = _lp().lp_lm_head_kl(*heads, m, y, dm, 7)
    assert np.array_equal(host(again[0]), got[0]) and np.array_equal(host(again[4]), got[4])
    # student backward
    lse_s, lse_t = to_dev(got[4]), to_dev(got[5])
    dH, dW = _lp().lp_lm_head_kl_backward(*heads, m, tile, lse_s, lse_t, to_dev(A["grad_kl"]))
    dH_o, dW_o = O.lm_head_kl_backward(*_wide(A), A["mask"], A["grad_kl"])
    for nm, g, w in (("dH", host(dH), dH_o), ("dW", host(dW), dW_o)):
        fro, mad = grad_errors(g, w)
        assert fro <= TOL_GRAD and mad <= TOL_GRAD, (nm, fro, mad)
    assert not host(dH)[~sc].any()


def test_kl_head_several_chunks_per_tile():
    """More scored rows than one chunk of the teacher buffer (4096 rows):
    a tile of 8192 rows runs as a full chunk plus a ragged one, in the
    forward and in the backward's dL/dlogits; rows match a run with one chunk
    per tile bitwise and the oracle to the fused tolerance."""
    A = _case(9000, 64, 128, 1000, seed=901, scored=0.7)
    heads = _dev_heads(A)
    m, y, dm = to_dev(A["mask"]), to_dev(A["targets"]), to_dev(A["diff_mask"])
    got = [host(t) for t in _lp().lp_lm_head_kl(*heads, m, y, dm, 8192)]
    want = O.lm_head_kl(*_wide(A), A["mask"], A["targets"], A["diff_mask"])
    sc = A["mask"] != 0
    for name, g, w in zip(("kl", "lp_s", "lp_t", "diff", "lse_s", "lse_t"), got, want):
        assert max_abs_err(g[sc], w[sc]) <= TOL_FWD, (name, max_abs_err(g[sc], w[sc]))
    small = [host(t) for t in _lp().lp_lm_head_kl(*heads, m, y, dm, 1000)]
    assert all(np.array_equal(a, b, equal_nan=True) for a, b in zip(got, small))
    lse_s, lse_t = to_dev(got[4]), to_dev(got[5])
    dH, dW = _lp().lp_lm_head_kl_backward(*heads, m, 8192, lse_s, lse_t, to_dev(A["grad_kl"]))
    dH_o, dW_o = O.lm_head_kl_backward(*_wide(A), A["mask"], A["grad_kl"])
    for nm, g, w in (("dH", host(dH), dH_o), ("dW", host(dW), dW_o)):
        fro, mad = grad_errors(g, w)
        assert fro <= TOL_GRAD and mad <= TOL_GRAD, (nm, fro, mad)


@pytest.mark.timeout(600)
def test_kl_backward_shipping_tile_elementwise():
    """Student gradients of the KL through the heads at the shipping tile
    size on the direct-to-LDS tiles: about 12,800 scored rows in tiles (and
    teacher-buffer chunks) of 4096 -- three full and a ragged fourth --,
    h = 256 for both heads, V = 5003.  Every element of dHidden and dW
    against the oracle."""
    T, h, V, tile = 16000, 256, 5003, 4096
    assert _lp().load().lp_lm_head_fast_tiles(T, h, V, h, h, tile, 1) == 1
    A = _case(T, h, h, V, seed=4097)
    n = int(A["mask"].sum())
    assert 3 * tile < n < 4 * tile, n
    heads = _dev_heads(A)
    m = to_dev(A["mask"])
    out = _lp().lp_lm_head_kl(*heads, m, None, None, tile)
    dH, dW = _lp().lp_lm_head_kl_backward(*heads, m, tile, out[4], out[5], to_dev(A["grad_kl"]))
    dH_o, dW_o = O.lm_head_kl_backward(*_wide(A), A["mask"], A["grad_kl"])
    for nm, g, w in (("dH", host(dH), dH_o), ("dW", host(dW), dW_o)):
        fro, mad = grad_errors(g, w)
        assert fro <= TOL_GRAD and mad <= TOL_GRAD, (nm, fro, mad)
    assert not host(dH)[A["mask"] == 0].any()


def test_kl_head_same_model_is_exactly_zero():
    A = _case(96, 128, 128, 777, seed=5, scored=1.0)
    hs, ws = to_dev_bits(A["student_hidden"], "bf16"), to_dev_bits(A["student_weight"], "bf16")
    kl, *_ = _lp().lp_lm_head_kl(hs, ws, hs, ws, None, None, None, 32)
    assert not host(kl).any()
    _, _, _, _, lse_s, lse_t = _lp().lp_lm_head_kl(hs, ws, hs, ws, None, None, None, 32)
    dH, dW = _lp().lp_lm_head_kl_backward(hs, ws, hs, ws, None, 32, lse_s, lse_t, to_dev(A["grad_kl"]))
    assert not host(dH).any() and not host(dW).any()


def test_kl_head_no_scored_rows_and_frozen_weight():
    A = _case(40, 64, 64, 300, seed=9, scored=0.0)
    heads = _dev_heads(A)
    m = to_dev(A["mask"])
    kl, lps, lpt, diff, lse_s, lse_t = _lp().lp_lm_head_kl(*heads, m, to_dev(A["targets"]), None, 16)
    assert not host(kl).any() and not host(lps).any() and not host(diff).any()
    dH, dW = _lp().lp_lm_head_kl_backward(*heads, m, 16, lse_s, lse_t, to_dev(A["grad_kl"]), need_grad_weight=False)
    assert dW is None and not host(dH).any()


class _LazyW:
    def __init__(self, bits):
        self.bits, self.shape = bits, bits.shape

    def __getitem__(self, sl):
        return O.widen_bf16(self.bits[sl])


@pytest.mark.timeout(900)
def test_kl_head_full_size_sampled():
    """T = 16384 rows, h = 7168 for both models, V = 129280, tile 4096 (the
    distillation workload): sampled rows of every forward output and of the
    student dHidden against the oracle; dW against the identity
    sum_v dW[v, :] = 0 (each row of p_u - p_v sums to 0)."""
    import torch
    cfg = synth.KLHeads(grads=True).build()
    A = cfg.arrays
    heads = _dev_heads(A)
    y, dm = to_dev(A["targets"]), to_dev(A["diff_mask"])
    out = _lp().lp_lm_head_kl(*heads, None, y, dm, cfg.tile_rows)
    got = [host(t) for t in out]
    rows = np.unique(np.concatenate([[0, 4095, 4096, cfg.T // 2, cfg.T - 1],
                                     np.random.default_rng(21).choice(cfg.T, 4, replace=False)]))
    want = O.lm_head_kl(O.widen_bf16(A["student_hidden"][rows]), _LazyW(A["student_weight"]),
                        O.widen_bf16(A["teacher_hidden"][rows]), _LazyW(A["teacher_weight"]), None,
                        A["targets"][rows], A["diff_mask"][rows])
    for name, g, w in zip(("kl", "lp_s", "lp_t", "diff", "lse_s", "lse_t"), got, want):
        assert max_abs_err(g[rows], w) <= TOL_FWD, (name, max_abs_err(g[rows], w))
    assert np.isfinite(got[0]).all() and (got[0] > -1e-3).all()
    g_kl = to_dev(A["grad_kl"])
    dH, dW = _lp().lp_lm_head_kl_backward(*heads, None, cfg.tile_rows, out[4], out[5], g_kl)
    Wl = _LazyW(A["student_weight"])
    _, dZ = O.lm_head_kl_logit_grad(O.widen_bf16(A["student_hidden"][rows]), Wl,
                                    O.widen_bf16(A["teacher_hidden"][rows]), _LazyW(A["teacher_weight"]), None,
                                    A["grad_kl"][rows])
    dH_o = np.zeros((len(rows), cfg.h))
    for j0 in range(0, cfg.V, 16384):
        dH_o += dZ[:, j0:j0 + 16384] @ Wl[j0:j0 + 16384]
    fro, mad = grad_errors(dH[torch.as_tensor(rows)].cpu().numpy(), dH_o)
    assert fro <= TOL_GRAD and mad <= TOL_GRAD, (fro, mad)
    colsum = dW.double().sum(0)
    scale = dW.double().abs().sum(0)
    assert torch.isfinite(dW).all().item()
    assert (colsum.abs() <= 1e-2 * scale).all().item()
    # dW summed over 4 tiles of 4096 against 8 tiles of 2048 (and 2 against 4 dW launches): a tile dropped,
    # doubled or paired with the wrong hidden rows would differ by far more than the summation order does
    _, dW2 = _lp().lp_lm_head_kl_backward(*heads, None, 2048, out[4], out[5], g_kl, need_grad_hidden=False)
    diff = (dW - dW2).double()
    rel_fro = (diff.norm() / dW2.double().norm()).item()
    rel_max = (diff.abs().max() / dW2.double().abs().max()).item()
    assert rel_fro <= TOL_GRAD and rel_max <= TOL_GRAD, (rel_fro, rel_max)


def test_kl_head_matches_kl_on_fp32_logits():
    """The KL through the heads against the KL on given logits fed each
    model's hidden @ W^T (fp64 product of the same bf16 values, rounded to
    fp32): the same fp32 reduction of the same logits."""
    A = _case(120, 64, 96, 2500, seed=77, scored=1.0)
    heads = _dev_heads(A)
    y = to_dev(A["targets"])
    kl_f, lps_f, lpt_f, _, _, _ = _lp().lp_lm_head_kl(*heads, None, y, None, 64)
    Hs, Ws, Ht, Wt = _wide(A)
    U = (Hs @ Ws.T).astype(np.float32)
    Vt = (Ht @ Wt.T).astype(np.float32)
    kl_l, lps_l, lpt_l, _ = _lp().lp_kl_full_vocab(to_dev(U), to_dev(Vt), y, None)
    assert max_abs_err(host(kl_f), host(kl_l)) <= 2e-5
    assert max_abs_err(host(lps_f), host(lps_l)) <= 2e-5 and max_abs_err(host(lpt_f), host(lpt_l)) <= 2e-5


def test_kl_head_extreme_logit_scales():
    """Logits in the hundreds (W ~ N(0, 4^2)): an unrelated teacher (KL in the
    tens) and a teacher that differs from the student in one weight row only
    (KL small while both logits are large: the cancellation case)."""
    T, h, V = 60, 64, 1200
    rng = np.random.default_rng(808)
    hs = synth.f32_to_bf16_bits(rng.normal(0, 1, size=(T, h)).astype(np.float32))
    ws = rng.normal(0, 4, size=(V, h)).astype(np.float32)
    for name, wt, ht in (("unrelated", rng.normal(0, 4, size=(V, h)).astype(np.float32), hs),
                         ("one row apart", ws.copy(), hs)):
        if name == "one row apart":
            wt[3] += rng.normal(0, 0.5, size=h).astype(np.float32)
        A = dict(student_hidden=hs, student_weight=synth.f32_to_bf16_bits(ws), teacher_hidden=ht,
                 teacher_weight=synth.f32_to_bf16_bits(wt))
        y = rng.integers(0, V, size=T).astype(np.int64)
        got = [host(t) for t in _lp().lp_lm_head_kl(*_dev_heads(A), None, to_dev(y), None, 16)]
        want = O.lm_head_kl(*_wide(A), None, y, None)
        kl, kl_o = got[0], want[0]
        assert np.all(np.isfinite(kl)) and np.all(kl > -1e-3), name
        assert np.all(np.abs(kl - kl_o) <= TOL_FWD + 2e-6 * np.abs(kl_o)), (name, np.abs(kl - kl_o).max())
        for g, w in zip(got[4:], want[4:]):  # both log-normalisers, in the hundreds
            assert np.all(np.abs(g - w) <= TOL_FWD + 2e-6 * np.abs(w)), name
