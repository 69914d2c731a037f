"""Python binding of liblp.so: per-token log-probs, entropy and exact KL over a
large vocabulary on MI355X.

Functions carry the C names (include/lp.h).  This layer only marshals
arguments: it checks dtypes, layouts, the length of every per-row array
(T, or T x K for the K-target calls) and that every tensor sits on the main
operand's device, all before anything is launched; it allocates outputs and
workspace with torch (device memory is all torch is used for) and passes raw
pointers plus the current HIP stream.  Every number is computed by the HIP
kernels; if liblp.so is missing, every call raises.
"""
from __future__ import annotations

from typing import Optional, Tuple

from . import _lib
from ._lib import LP_BF16, LP_FP16, LP_FP32, LPError, check, load

__all__ = [
    "lp_logprobs_entropy", "lp_lm_head_logprobs_entropy", "lp_lm_head_logprobs_entropy_backward",
    "lp_lm_head_workspace_bytes", "lp_kl_full_vocab", "lp_prob_diff", "lp_version", "lp_timing_enable",
    "lp_timing_read", "lp_timing_clock", "lp_logprobs_entropy_k", "lp_lm_head_logprobs_entropy_k",
    "lp_lm_head_logprobs_entropy_backward_k", "lp_prob_diff_stats", "lp_lm_head_kl_workspace_bytes",
    "lp_lm_head_kl", "lp_lm_head_kl_backward", "LPError", "load",
]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LP_BF16
    if t.dtype == torch.float16:
        return LP_FP16
    if t.dtype == torch.float32:
        return LP_FP32
    raise TypeError(f"unsupported logits dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t, name):
    if t is not None and not t.is_cuda:
        raise ValueError(f"{name} must be a device (GPU) tensor")


def _on(device, **tensors):
    """Every given tensor lives on `device` (checked after all shapes, so a
    wrong length is reported as such even for host tensors)."""
    for name, t in tensors.items():
        if t is None:
            continue
        _dev(t, name)
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _rows(t, name):
    """2-D tensor with unit stride along columns; returns its leading dimension."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


def _vec(t, name, dtype=None, n=None):
    """Contiguous tensor of `dtype` (bool accepted for uint8) holding exactly
    `n` elements when n is given: a short per-row array would be read past
    its end by the kernels, so it is refused here."""
    if t is None:
        return None
    torch = _torch()
    if dtype is not None and t.dtype != dtype:
        if dtype == torch.uint8 and t.dtype == torch.bool:
            t = t.view(torch.uint8)
        else:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {t.numel()}")
    return t


def _bf16_2d(t, name):
    torch = _torch()
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    return t


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def lp_version() -> int:
    return load().lp_version()


def lp_timing_enable(on) -> None:
    """Start (clearing old records) or stop per-kernel HIP-event timing; 2 also
    samples the fused forward GEMM's shader clock (lp_timing_clock)."""
    load().lp_timing_enable(2 if on == 2 else (1 if on else 0))


def lp_timing_clock(kernel: str = "k_fwd_tile"):
    """(mean shader clock in MHz, workgroups sampled) of the last sampled launch."""
    import ctypes
    mhz = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    check("lp_timing_clock", load().lp_timing_clock(kernel.encode(), ctypes.byref(mhz), ctypes.byref(n)))
    return float(mhz.value), int(n.value)


def lp_timing_read(kernel: str):
    """(launches, total_ms) recorded for `kernel` since timing was enabled."""
    import ctypes
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    check("lp_timing_read", load().lp_timing_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def lp_logprobs_entropy(logits, targets, mask=None, temperature: float = 1.0, chunk_rows: int = -1, *,
                        want_entropy: bool = True, logprob=None, entropy=None, stream=None):
    """(logprob[T], entropy[T] or None) of model-precision logits [T, V]."""
    torch = _torch()
    lib = load()
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [T, V]")
    T, V = logits.shape
    ld = _rows(logits, "logits")
    targets = _vec(targets, "targets", torch.int64, T)
    mask = _vec(mask, "mask", torch.uint8, T)
    logprob = _vec(logprob, "logprob", torch.float32, T)
    entropy = _vec(entropy, "entropy", torch.float32, T)
    _on(logits.device, logits=logits, targets=targets, mask=mask, logprob=logprob, entropy=entropy)
    if logprob is None:
        logprob = torch.empty(T, dtype=torch.float32, device=logits.device)
    if want_entropy and entropy is None:
        entropy = torch.empty(T, dtype=torch.float32, device=logits.device)
    st = lib.lp_logprobs_entropy(_ptr(logits), _dtype_code(logits), T, V, ld, _ptr(targets), _ptr(mask),
                                 float(temperature), int(chunk_rows), _ptr(logprob), _ptr(entropy), _stream(stream))
    check("lp_logprobs_entropy", st)
    return logprob, entropy


def lp_lm_head_workspace_bytes(T: int, h: int, V: int, tile_rows: int, backward: bool) -> int:
    return int(load().lp_lm_head_workspace_bytes(T, h, V, tile_rows, 1 if backward else 0))


def _workspace(nbytes: int, device, workspace):
    """(tensor, size in bytes): the caller's workspace after checks, or a new one."""
    torch = _torch()
    if workspace is not None:
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        _on(device, workspace=workspace)
        size = workspace.numel() * workspace.element_size()
        if size < nbytes:
            raise ValueError(f"workspace too small: {size} bytes, {nbytes} needed")
        return workspace, size
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel()


def _lm_head_operands(hidden, weight):
    """(T, h, V) of bf16 hidden [T, h] and weight [V, h]."""
    _bf16_2d(hidden, "hidden")
    _bf16_2d(weight, "weight")
    T, h = hidden.shape
    V, h2 = weight.shape
    if h2 != h:
        raise ValueError("hidden and weight disagree on h")
    return T, h, V


def lp_lm_head_logprobs_entropy(hidden, weight, targets, mask=None, temperature: float = 1.0,
                                tile_rows: int = 4096, *, want_entropy: bool = True, want_lse: bool = True,
                                workspace=None, stream=None):
    """(logprob, entropy, lse) of softmax(hidden @ weight^T / temperature); bf16 hidden [T, h], weight [V, h]."""
    torch = _torch()
    lib = load()
    T, h, V = _lm_head_operands(hidden, weight)
    ld_h, ld_w = _rows(hidden, "hidden"), _rows(weight, "weight")
    targets = _vec(targets, "targets", torch.int64, T)
    mask = _vec(mask, "mask", torch.uint8, T)
    dev = hidden.device
    _on(dev, hidden=hidden, weight=weight, targets=targets, mask=mask)
    lp = torch.empty(T, dtype=torch.float32, device=dev)
    H = torch.empty(T, dtype=torch.float32, device=dev) if want_entropy else None
    lse = torch.empty(T, dtype=torch.float32, device=dev) if want_lse else None
    ws, ws_bytes = _workspace(lp_lm_head_workspace_bytes(T, h, V, tile_rows, False), dev, workspace)
    st = lib.lp_lm_head_logprobs_entropy(_ptr(hidden), ld_h, _ptr(weight), ld_w, T, h, V, _ptr(targets), _ptr(mask),
                                         float(temperature), int(tile_rows), _ptr(lp), _ptr(H), _ptr(lse), _ptr(ws),
                                         ws_bytes, _stream(stream))
    check("lp_lm_head_logprobs_entropy", st)
    return lp, H, lse


def lp_lm_head_logprobs_entropy_backward(hidden, weight, targets, mask, temperature: float, tile_rows: int,
                                         lse, entropy, grad_logprob, grad_entropy=None, *,
                                         need_grad_hidden: bool = True, need_grad_weight: bool = True,
                                         workspace=None, stream=None) -> Tuple:
    """(grad_hidden fp32 [T, h] or None, grad_weight fp32 [V, h] or None)."""
    torch = _torch()
    lib = load()
    T, h, V = _lm_head_operands(hidden, weight)
    ld_h, ld_w = _rows(hidden, "hidden"), _rows(weight, "weight")
    targets = _vec(targets, "targets", torch.int64, T)
    mask = _vec(mask, "mask", torch.uint8, T)
    lse = _vec(lse, "lse", torch.float32, T)
    entropy = _vec(entropy, "entropy", torch.float32, T)
    grad_logprob = _vec(grad_logprob, "grad_logprob", torch.float32, T)
    grad_entropy = _vec(grad_entropy, "grad_entropy", torch.float32, T)
    dev = hidden.device
    _on(dev, hidden=hidden, weight=weight, targets=targets, mask=mask, lse=lse, entropy=entropy,
        grad_logprob=grad_logprob, grad_entropy=grad_entropy)
    dH = torch.empty((T, h), dtype=torch.float32, device=dev) if need_grad_hidden else None
    dW = torch.empty((V, h), dtype=torch.float32, device=dev) if need_grad_weight else None
    ws, ws_bytes = _workspace(lp_lm_head_workspace_bytes(T, h, V, tile_rows, True), dev, workspace)
    st = lib.lp_lm_head_logprobs_entropy_backward(
        _ptr(hidden), ld_h, _ptr(weight), ld_w, T, h, V, _ptr(targets), _ptr(mask), float(temperature),
        int(tile_rows), _ptr(lse), _ptr(entropy), _ptr(grad_logprob), _ptr(grad_entropy), _ptr(dH), _ptr(dW),
        _ptr(ws), ws_bytes, _stream(stream))
    check("lp_lm_head_logprobs_entropy_backward", st)
    return dH, dW


def lp_kl_full_vocab(student, teacher, targets=None, diff_mask=None, *, want_target_logprobs: bool = True,
                     stream=None):
    """(kl, lp_student, lp_teacher, prob_diff); the last three are None without targets."""
    torch = _torch()
    lib = load()
    if student.dtype != teacher.dtype or student.shape != teacher.shape or student.dim() != 2:
        raise ValueError("student and teacher must be 2-D with the same dtype and shape")
    T, V = student.shape
    ld_s, ld_t = _rows(student, "student"), _rows(teacher, "teacher")
    targets = _vec(targets, "targets", torch.int64, T)
    diff_mask = _vec(diff_mask, "diff_mask", torch.uint8, T)
    dev = student.device
    _on(dev, student=student, teacher=teacher, targets=targets, diff_mask=diff_mask)
    kl = torch.empty(T, dtype=torch.float32, device=dev)
    lps = lpt = diff = None
    if targets is not None and want_target_logprobs:
        lps = torch.empty(T, dtype=torch.float32, device=dev)
        lpt = torch.empty(T, dtype=torch.float32, device=dev)
        diff = torch.empty(T, dtype=torch.float32, device=dev)
    st = lib.lp_kl_full_vocab(_ptr(student), _ptr(teacher), _dtype_code(student), T, V, ld_s, ld_t, _ptr(kl),
                              _ptr(targets), _ptr(diff_mask), _ptr(lps), _ptr(lpt), _ptr(diff), _stream(stream))
    check("lp_kl_full_vocab", st)
    return kl, lps, lpt, diff


def lp_prob_diff(lp_a, lp_b, mask=None, *, out=None, stream=None):
    """mask * |exp(lp_a) - exp(lp_b)| elementwise (fp32 vectors)."""
    torch = _torch()
    lib = load()
    lp_a = _vec(lp_a, "lp_a", torch.float32)
    n = lp_a.numel()
    lp_b = _vec(lp_b, "lp_b", torch.float32, n)
    mask = _vec(mask, "mask", torch.uint8, n)
    out = _vec(out, "out", torch.float32, n)
    _on(lp_a.device, lp_a=lp_a, lp_b=lp_b, mask=mask, out=out)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=lp_a.device)
    st = lib.lp_prob_diff(_ptr(lp_a), _ptr(lp_b), _ptr(mask), n, _ptr(out), _stream(stream))
    check("lp_prob_diff", st)
    return out


def _targets_k(targets, T):
    torch = _torch()
    t = _vec(targets, "targets", torch.int64)
    if t is None or t.dim() != 2 or t.size(0) != T:
        raise ValueError("targets must be [T, K]")
    return t, t.size(1)


def lp_logprobs_entropy_k(logits, targets, mask=None, temperature: float = 1.0, chunk_rows: int = -1, *,
                          want_entropy: bool = True, stream=None):
    """(logprob [T, K], entropy [T] or None) with K targets per row (targets [T, K] int64)."""
    torch = _torch()
    lib = load()
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [T, V]")
    T, V = logits.shape
    ld = _rows(logits, "logits")
    targets, K = _targets_k(targets, T)
    mask = _vec(mask, "mask", torch.uint8, T)
    _on(logits.device, logits=logits, targets=targets, mask=mask)
    lp = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    H = torch.empty(T, dtype=torch.float32, device=logits.device) if want_entropy else None
    st = lib.lp_logprobs_entropy_k(_ptr(logits), _dtype_code(logits), T, V, ld, _ptr(targets), K, _ptr(mask),
                                   float(temperature), int(chunk_rows), _ptr(lp), _ptr(H), _stream(stream))
    check("lp_logprobs_entropy_k", st)
    return lp, H


def lp_lm_head_logprobs_entropy_k(hidden, weight, targets, mask=None, temperature: float = 1.0,
                                  tile_rows: int = 4096, *, workspace=None, stream=None):
    """(logprob [T, K], entropy [T], lse [T]) of the fused LM head with K targets per row."""
    torch = _torch()
    lib = load()
    T, h, V = _lm_head_operands(hidden, weight)
    ld_h, ld_w = _rows(hidden, "hidden"), _rows(weight, "weight")
    targets, K = _targets_k(targets, T)
    mask = _vec(mask, "mask", torch.uint8, T)
    dev = hidden.device
    _on(dev, hidden=hidden, weight=weight, targets=targets, mask=mask)
    lp = torch.empty((T, K), dtype=torch.float32, device=dev)
    H = torch.empty(T, dtype=torch.float32, device=dev)
    lse = torch.empty(T, dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(lp_lm_head_workspace_bytes(T, h, V, tile_rows, False), dev, workspace)
    st = lib.lp_lm_head_logprobs_entropy_k(_ptr(hidden), ld_h, _ptr(weight), ld_w, T, h, V, _ptr(targets), K,
                                           _ptr(mask), float(temperature), int(tile_rows), _ptr(lp), _ptr(H),
                                           _ptr(lse), _ptr(ws), ws_bytes, _stream(stream))
    check("lp_lm_head_logprobs_entropy_k", st)
    return lp, H, lse


def lp_lm_head_logprobs_entropy_backward_k(hidden, weight, targets, mask, temperature: float, tile_rows: int,
                                           lse, entropy, grad_logprob, grad_entropy=None, *,
                                           need_grad_hidden: bool = True, need_grad_weight: bool = True,
                                           workspace=None, stream=None):
    """Backward of the K-target fused LM head; grad_logprob is [T, K]."""
    torch = _torch()
    lib = load()
    T, h, V = _lm_head_operands(hidden, weight)
    ld_h, ld_w = _rows(hidden, "hidden"), _rows(weight, "weight")
    targets, K = _targets_k(targets, T)
    mask = _vec(mask, "mask", torch.uint8, T)
    lse = _vec(lse, "lse", torch.float32, T)
    entropy = _vec(entropy, "entropy", torch.float32, T)
    grad_logprob = _vec(grad_logprob, "grad_logprob", torch.float32, T * K)
    if grad_logprob is None or grad_logprob.shape != (T, K):
        raise ValueError("grad_logprob must be [T, K]")
    grad_entropy = _vec(grad_entropy, "grad_entropy", torch.float32, T)
    dev = hidden.device
    _on(dev, hidden=hidden, weight=weight, targets=targets, mask=mask, lse=lse, entropy=entropy,
        grad_logprob=grad_logprob, grad_entropy=grad_entropy)
    dH = torch.empty((T, h), dtype=torch.float32, device=dev) if need_grad_hidden else None
    dW = torch.empty((V, h), dtype=torch.float32, device=dev) if need_grad_weight else None
    ws, ws_bytes = _workspace(lp_lm_head_workspace_bytes(T, h, V, tile_rows, True), dev, workspace)
    st = lib.lp_lm_head_logprobs_entropy_backward_k(
        _ptr(hidden), ld_h, _ptr(weight), ld_w, T, h, V, _ptr(targets), K, _ptr(mask), float(temperature),
        int(tile_rows), _ptr(lse), _ptr(entropy), _ptr(grad_logprob), _ptr(grad_entropy), _ptr(dH), _ptr(dW),
        _ptr(ws), ws_bytes, _stream(stream))
    check("lp_lm_head_logprobs_entropy_backward_k", st)
    return dH, dW


def lp_prob_diff_stats(lp_a, lp_b, mask=None, *, stream=None):
    """Device float64 [5]: count, max, mean, std of mask * |exp(a) - exp(b)| and Pearson(exp(a), exp(b))."""
    torch = _torch()
    lib = load()
    lp_a = _vec(lp_a, "lp_a", torch.float32)
    n = lp_a.numel()
    lp_b = _vec(lp_b, "lp_b", torch.float32, n)
    mask = _vec(mask, "mask", torch.uint8, n)
    _on(lp_a.device, lp_a=lp_a, lp_b=lp_b, mask=mask)
    out = torch.empty(5, dtype=torch.float64, device=lp_a.device)
    ws = torch.empty(max(int(lib.lp_prob_diff_stats_workspace_bytes()), 256), dtype=torch.uint8, device=lp_a.device)
    st = lib.lp_prob_diff_stats(_ptr(lp_a), _ptr(lp_b), _ptr(mask), n, _ptr(out), _ptr(ws), ws.numel(),
                                _stream(stream))
    check("lp_prob_diff_stats", st)
    return out


def lp_lm_head_kl_workspace_bytes(T: int, h_student: int, V: int, tile_rows: int, backward: bool) -> int:
    return int(load().lp_lm_head_kl_workspace_bytes(T, h_student, V, tile_rows, 1 if backward else 0))


def _heads(student_hidden, student_weight, teacher_hidden, teacher_weight):
    for t, n in ((student_hidden, "student_hidden"), (student_weight, "student_weight"),
                 (teacher_hidden, "teacher_hidden"), (teacher_weight, "teacher_weight")):
        _bf16_2d(t, n)
    T, hs = student_hidden.shape
    V, hs2 = student_weight.shape
    T2, ht = teacher_hidden.shape
    V2, ht2 = teacher_weight.shape
    if hs2 != hs or ht2 != ht or T2 != T or V2 != V:
        raise ValueError("student / teacher hidden and weight shapes disagree")
    args = [_ptr(student_hidden), _rows(student_hidden, "student_hidden"), _ptr(student_weight),
            _rows(student_weight, "student_weight"), hs, _ptr(teacher_hidden), _rows(teacher_hidden, "teacher_hidden"),
            _ptr(teacher_weight), _rows(teacher_weight, "teacher_weight"), ht]
    tensors = dict(student_hidden=student_hidden, student_weight=student_weight, teacher_hidden=teacher_hidden,
                   teacher_weight=teacher_weight)
    return T, V, hs, ht, args, tensors


def lp_lm_head_kl(student_hidden, student_weight, teacher_hidden, teacher_weight, mask=None, targets=None,
                  diff_mask=None, tile_rows: int = 4096, *, want_lse: bool = True, workspace=None, stream=None):
    """(kl, lp_student, lp_teacher, prob_diff, lse_student, lse_teacher) of the logits hidden @ W^T of each
    model (bf16 hiddens [T, h_*], weights [V, h_*]); the target outputs are None without targets."""
    torch = _torch()
    lib = load()
    T, V, hs, ht, head_args, heads = _heads(student_hidden, student_weight, teacher_hidden, teacher_weight)
    mask = _vec(mask, "mask", torch.uint8, T)
    targets = _vec(targets, "targets", torch.int64, T)
    diff_mask = _vec(diff_mask, "diff_mask", torch.uint8, T)
    dev = student_hidden.device
    _on(dev, **heads, mask=mask, targets=targets, diff_mask=diff_mask)
    f32 = dict(dtype=torch.float32, device=dev)
    kl = torch.empty(T, **f32)
    lps = lpt = diff = None
    if targets is not None:
        lps, lpt, diff = torch.empty(T, **f32), torch.empty(T, **f32), torch.empty(T, **f32)
    lseu = torch.empty(T, **f32) if want_lse else None
    lsev = torch.empty(T, **f32) if want_lse else None
    ws, ws_bytes = _workspace(lp_lm_head_kl_workspace_bytes(T, hs, V, tile_rows, False), dev, workspace)
    st = lib.lp_lm_head_kl(*head_args, T, V, _ptr(mask), _ptr(targets), _ptr(diff_mask), int(tile_rows), _ptr(kl),
                           _ptr(lps), _ptr(lpt), _ptr(diff), _ptr(lseu), _ptr(lsev), _ptr(ws), ws_bytes,
                           _stream(stream))
    check("lp_lm_head_kl", st)
    return kl, lps, lpt, diff, lseu, lsev


def lp_lm_head_kl_backward(student_hidden, student_weight, teacher_hidden, teacher_weight, mask, tile_rows: int,
                           lse_student, lse_teacher, grad_kl, *, need_grad_hidden: bool = True,
                           need_grad_weight: bool = True, workspace=None, stream=None) -> Tuple:
    """(grad_hidden fp32 [T, h_student] or None, grad_weight fp32 [V, h_student] or None) of sum_t g_t KL_t."""
    torch = _torch()
    lib = load()
    T, V, hs, ht, head_args, heads = _heads(student_hidden, student_weight, teacher_hidden, teacher_weight)
    mask = _vec(mask, "mask", torch.uint8, T)
    lse_student = _vec(lse_student, "lse_student", torch.float32, T)
    lse_teacher = _vec(lse_teacher, "lse_teacher", torch.float32, T)
    grad_kl = _vec(grad_kl, "grad_kl", torch.float32, T)
    dev = student_hidden.device
    _on(dev, **heads, mask=mask, lse_student=lse_student, lse_teacher=lse_teacher, grad_kl=grad_kl)
    dH = torch.empty((T, hs), dtype=torch.float32, device=dev) if need_grad_hidden else None
    dW = torch.empty((V, hs), dtype=torch.float32, device=dev) if need_grad_weight else None
    ws, ws_bytes = _workspace(lp_lm_head_kl_workspace_bytes(T, hs, V, tile_rows, True), dev, workspace)
    st = lib.lp_lm_head_kl_backward(*head_args, T, V, _ptr(mask), int(tile_rows), _ptr(lse_student),
                                    _ptr(lse_teacher), _ptr(grad_kl), _ptr(dH), _ptr(dW), _ptr(ws), ws_bytes,
                                    _stream(stream))
    check("lp_lm_head_kl_backward", st)
    return dH, dW
