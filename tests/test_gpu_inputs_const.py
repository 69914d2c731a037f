"""Every entry point treats its inputs as read-only: after each call (forward,
backward, K targets, both KL paths, the prob diff and its aggregates) every
input buffer holds the same bytes as before.  The prior art's cross-entropy
works in place on its logits; this library's contract is that it never does."""
import numpy as np
import pytest

import synth
from tests.helpers import to_dev, to_dev_bits

pytestmark = pytest.mark.gpu


def _lp():
    import entropy_chunked_row_amd as lp
    return lp


def _snap(ts):
    import torch
    return [None if t is None else t.detach().clone() for t in ts]


def _same(before, after):
    import torch
    for i, (b, a) in enumerate(zip(before, after)):
        if b is None:
            continue
        assert torch.equal(b.view(torch.uint8), a.view(torch.uint8)), f"input {i} changed"


def _check(call, *inputs):
    before = _snap(inputs)
    call(*inputs)
    import torch
    torch.cuda.synchronize()
    _same(before, inputs)


def test_every_entry_point_leaves_its_inputs_unchanged():
    rng = np.random.default_rng(77)
    T, h, V, K, tile = 200, 128, 3001, 3, 64
    bf = lambda a: to_dev_bits(synth.f32_to_bf16_bits(a.astype(np.float32)), "bf16")
    hid = bf(rng.normal(0, 1, (T, h)))
    W = bf(rng.normal(0, 0.05, (V, h)))
    hid_t = bf(rng.normal(0, 1, (T, 96)))
    W_t = bf(rng.normal(0, 0.05, (V, 96)))
    logits = bf(rng.normal(0, 3, (T, V)))
    logits16 = to_dev_bits(rng.normal(0, 4, (T, V)).astype(np.float16).view(np.uint16), "fp16")
    teacher16 = to_dev_bits(rng.normal(0, 4, (T, V)).astype(np.float16).view(np.uint16), "fp16")
    y = to_dev(rng.integers(0, V, T).astype(np.int64))
    yk = to_dev(rng.integers(0, V, (T, K)).astype(np.int64))
    m = to_dev((rng.random(T) < 0.7).astype(np.uint8))
    dm = to_dev((rng.random(T) < 0.5).astype(np.uint8))
    g = to_dev(rng.normal(0, 1, T).astype(np.float32))
    gk = to_dev(rng.normal(0, 1, (T, K)).astype(np.float32))
    gh = to_dev(rng.normal(0, 0.1, T).astype(np.float32))
    lp = _lp()

    _check(lambda x, t, mk: lp.lp_logprobs_entropy(x, t, mk, 0.7, 64), logits, y, m)
    _check(lambda x, t, mk: lp.lp_logprobs_entropy_k(x, t, mk, 0.7, 64), logits, yk, m)

    _, H, lse = lp.lp_lm_head_logprobs_entropy(hid, W, y, m, 0.7, tile)
    _check(lambda a, b, t, mk: lp.lp_lm_head_logprobs_entropy(a, b, t, mk, 0.7, tile), hid, W, y, m)
    _check(lambda a, b, t, mk, l, e, gl, ge: lp.lp_lm_head_logprobs_entropy_backward(a, b, t, mk, 0.7, tile, l, e,
                                                                                     gl, ge),
           hid, W, y, m, lse, H, g, gh)

    _, Hk, lsek = lp.lp_lm_head_logprobs_entropy_k(hid, W, yk, m, 0.7, tile)
    _check(lambda a, b, t, mk: lp.lp_lm_head_logprobs_entropy_k(a, b, t, mk, 0.7, tile), hid, W, yk, m)
    _check(lambda a, b, t, mk, l, e, gl, ge: lp.lp_lm_head_logprobs_entropy_backward_k(a, b, t, mk, 0.7, tile, l, e,
                                                                                       gl, ge),
           hid, W, yk, m, lsek, Hk, gk, gh)

    kl, lps, lpt, _ = lp.lp_kl_full_vocab(logits16, teacher16, y, dm)
    _check(lambda u, v, t, d: lp.lp_kl_full_vocab(u, v, t, d), logits16, teacher16, y, dm)
    _check(lambda a, b, d: lp.lp_prob_diff(a, b, d), lps, lpt, dm)
    _check(lambda a, b, d: lp.lp_prob_diff_stats(a, b, d), lps, lpt, dm)

    out = lp.lp_lm_head_kl(hid, W, hid_t, W_t, m, y, dm, tile)
    _check(lambda a, b, c, d, mk, t, dd: lp.lp_lm_head_kl(a, b, c, d, mk, t, dd, tile), hid, W, hid_t, W_t, m, y, dm)
    _check(lambda a, b, c, d, mk, lu, lv, gg: lp.lp_lm_head_kl_backward(a, b, c, d, mk, tile, lu, lv, gg),
           hid, W, hid_t, W_t, m, out[4], out[5], g)
