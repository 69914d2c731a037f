"""CPU checks of the Python binding's argument marshalling: every per-row
array must hold exactly T (or T x K) elements and sit on the main operand's
device, and both are refused with ValueError before anything reaches the
library.  Host tensors are enough: the length checks run before the device
checks, and nothing here is launched."""
import pytest
import torch

import entropy_chunked_row_amd as lp

T, V, H = 6, 32, 16


def _i64(n):
    return torch.zeros(n, dtype=torch.int64)


def _f32(n):
    return torch.zeros(n, dtype=torch.float32)


def _u8(n):
    return torch.ones(n, dtype=torch.uint8)


def _bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def _calls(short):
    """(name, callable) for every wrapper, with the per-row array `short`
    given T - 1 elements (or T x K - 1) and every other array sized right."""
    n = {k: (T - 1 if k == short else T) for k in
         ("targets", "mask", "lse", "entropy", "grad_logprob", "grad_entropy", "diff_mask", "grad_kl", "lse_student",
          "lse_teacher", "logprob", "lp_b", "out")}
    logits = _bf16(T, V)
    hid, W = _bf16(T, H), _bf16(V, H)
    yield "lp_logprobs_entropy", lambda: lp.lp_logprobs_entropy(
        logits, _i64(n["targets"]), _u8(n["mask"]), 0.7, 2, logprob=_f32(n["logprob"]))
    yield "lp_lm_head_logprobs_entropy", lambda: lp.lp_lm_head_logprobs_entropy(
        hid, W, _i64(n["targets"]), _u8(n["mask"]), 1.0, 4)
    yield "lp_lm_head_logprobs_entropy_backward", lambda: lp.lp_lm_head_logprobs_entropy_backward(
        hid, W, _i64(n["targets"]), _u8(n["mask"]), 1.0, 4, _f32(n["lse"]), _f32(n["entropy"]),
        _f32(n["grad_logprob"]), _f32(n["grad_entropy"]))
    yield "lp_kl_full_vocab", lambda: lp.lp_kl_full_vocab(logits, logits, _i64(n["targets"]), _u8(n["diff_mask"]))
    yield "lp_lm_head_kl", lambda: lp.lp_lm_head_kl(hid, W, hid, W, _u8(n["mask"]), _i64(n["targets"]),
                                                    _u8(n["diff_mask"]), 4)
    yield "lp_lm_head_kl_backward", lambda: lp.lp_lm_head_kl_backward(
        hid, W, hid, W, _u8(n["mask"]), 4, _f32(n["lse_student"]), _f32(n["lse_teacher"]), _f32(n["grad_kl"]))
    yield "lp_prob_diff", lambda: lp.lp_prob_diff(_f32(T), _f32(n["lp_b"]), _u8(n["mask"]), out=_f32(n["out"]))
    yield "lp_prob_diff_stats", lambda: lp.lp_prob_diff_stats(_f32(T), _f32(n["lp_b"]), _u8(n["mask"]))


SHORTS = {
    "lp_logprobs_entropy": ("targets", "mask", "logprob"),
    "lp_lm_head_logprobs_entropy": ("targets", "mask"),
    "lp_lm_head_logprobs_entropy_backward": ("targets", "mask", "lse", "entropy", "grad_logprob", "grad_entropy"),
    "lp_kl_full_vocab": ("targets", "diff_mask"),
    "lp_lm_head_kl": ("mask", "targets", "diff_mask"),
    "lp_lm_head_kl_backward": ("mask", "lse_student", "lse_teacher", "grad_kl"),
    "lp_prob_diff": ("lp_b", "mask", "out"),
    "lp_prob_diff_stats": ("lp_b", "mask"),
}


@pytest.mark.parametrize("fn,short", [(f, s) for f, ss in SHORTS.items() for s in ss])
def test_short_per_row_array_is_refused(fn, short):
    call = dict(_calls(short))[fn]
    with pytest.raises(ValueError, match="elements"):
        call()


@pytest.mark.parametrize("fn", sorted(SHORTS))
def test_host_tensors_are_refused_after_the_length_checks(fn):
    """With every length right, the next check is placement: host tensors
    never reach the library."""
    call = dict(_calls(None))[fn]
    with pytest.raises(ValueError, match="device"):
        call()


def test_k_target_calls_check_shapes():
    logits = _bf16(T, V)
    hid, W = _bf16(T, H), _bf16(V, H)
    y = _i64(T * 3).view(T, 3)
    with pytest.raises(ValueError, match="targets must be"):
        lp.lp_logprobs_entropy_k(logits, _i64(T * 3).view(3, T))
    with pytest.raises(ValueError, match="mask"):
        lp.lp_logprobs_entropy_k(logits, y, _u8(T + 1))
    with pytest.raises(ValueError, match="grad_logprob"):
        lp.lp_lm_head_logprobs_entropy_backward_k(hid, W, y, None, 1.0, 4, _f32(T), _f32(T), _f32(T))
    with pytest.raises(ValueError, match="lse"):
        lp.lp_lm_head_logprobs_entropy_backward_k(hid, W, y, None, 1.0, 4, _f32(T - 1), _f32(T), _f32(T * 3))


def test_dtypes_and_workspace_are_checked():
    hid, W = _bf16(T, H), _bf16(V, H)
    with pytest.raises(TypeError, match="bfloat16"):
        lp.lp_lm_head_logprobs_entropy_backward(hid.float(), W, _i64(T), None, 1.0, 4, _f32(T), _f32(T), _f32(T))
    with pytest.raises(TypeError, match="int64"):
        lp.lp_lm_head_logprobs_entropy(hid, W, _f32(T), None)
    # a caller's workspace must be large enough, counted in bytes whatever its dtype
    with pytest.raises(ValueError, match="device|workspace"):
        lp.lp_lm_head_logprobs_entropy(hid, W, _i64(T), None, workspace=torch.zeros(4, dtype=torch.float32))
