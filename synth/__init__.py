"""Seeded synthetic inputs shared by the oracle-side tests and the GPU side.

This module only draws random numbers and rounds them to the model precision
the library consumes (bf16 / fp16 bit patterns); it holds none of the method's
arithmetic.  Every array is produced on the host so that the oracle and the
kernels see identical bits.

Streams: numpy PCG64 seeded with SeedSequence([ROOT_SEED, workload_id,
stream_id, block_id]).  Large arrays are filled in fixed row blocks (the block
layout depends only on the shape), one independent stream per block, so the
bytes do not depend on how many threads fill them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20261202

# stream ids
S_VALUES, S_TARGETS, S_MASK, S_SPIKE, S_WEIGHT, S_NOISE, S_GRAD_LP, S_GRAD_H, S_NOISE_W, S_GRAD_KL = range(10)

_BLOCK_ELEMS = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(workload: int, stream: int, block: int = 0, seed: int = ROOT_SEED) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, workload, stream, block])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs are finite draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _row_blocks(rows: int, cols: int):
    per = max(1, _BLOCK_ELEMS // max(1, cols))
    return [(r0, min(rows, r0 + per)) for r0 in range(0, rows, per)]


def normal_bits(shape, sigma: float, precision: str, workload: int, stream: int,
                seed: int = ROOT_SEED, row_hook=None) -> np.ndarray:
    """N(0, sigma^2) drawn in fp32, rounded to `precision` ('bf16'|'fp16'),
    returned as uint16 bits.  `row_hook(r0, r1, block_f32)` may edit a block
    in fp32 before rounding (used for target spikes)."""
    rows, cols = shape
    out = np.empty((rows, cols), dtype=np.uint16)
    conv = f32_to_bf16_bits if precision == "bf16" else f32_to_fp16_bits

    def fill(ib):
        i, (r0, r1) = ib
        g = rng(workload, stream, i, seed)
        blk = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        if sigma != 1.0:
            blk *= np.float32(sigma)
        if row_hook is not None:
            row_hook(r0, r1, blk)
        out[r0:r1] = conv(blk)

    blocks = list(enumerate(_row_blocks(rows, cols)))
    if len(blocks) == 1:
        fill(blocks[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, blocks))
    return out


def normal_f32(n: int, sigma: float, workload: int, stream: int, seed: int = ROOT_SEED) -> np.ndarray:
    g = rng(workload, stream, 0, seed)
    return (g.standard_normal(n, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def uniform_targets(T: int, V: int, workload: int, seed: int = ROOT_SEED) -> np.ndarray:
    return rng(workload, S_TARGETS, 0, seed).integers(0, V, size=T, dtype=np.int64)


def packed_response_mask(T: int, len_lo: int, len_hi: int, prompt_frac: float,
                         workload: int, seed: int = ROOT_SEED) -> np.ndarray:
    """Sequences of length U{len_lo..len_hi} packed back to back until T rows
    are filled (the last one is cut).  The first floor(prompt_frac * L) rows of
    each sequence are prompt (0), the rest response (1)."""
    g = rng(workload, S_MASK, 0, seed)
    mask = np.zeros(T, dtype=np.uint8)
    pos = 0
    while pos < T:
        L = int(g.integers(len_lo, len_hi + 1))
        n_prompt = int(np.floor(prompt_frac * L))
        end = min(T, pos + L)
        mask[min(T, pos + n_prompt):end] = 1
        pos += L
    return mask


def bernoulli_mask(T: int, p: float, workload: int, seed: int = ROOT_SEED) -> np.ndarray:
    return (rng(workload, S_MASK, 0, seed).random(T) < p).astype(np.uint8)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

W_TINY_LM_HEAD, W_LOGITS, W_LM_HEAD_FWD, W_KL, W_LM_HEAD_BWD, W_KL_HEADS = 1, 2, 3, 4, 5, 6


@dataclass
class LogitsInput:
    """bf16/fp16 logits [T, V] ~ N(0, sigma^2) with a +spike at the target on a
    fraction of rows; packed response mask; temperature; chunk rows."""
    T: int = 8192
    V: int = 151936
    sigma: float = 3.0
    spike: float = 8.0
    spike_frac: float = 0.30
    run_lo: int = 256
    run_hi: int = 2048
    prompt_frac: float = 0.25
    temperature: float = 0.7
    chunk_rows: int = 4096
    precision: str = "bf16"
    seed: int = ROOT_SEED
    arrays: dict = field(default_factory=dict, repr=False)

    def build(self):
        T, V = self.T, self.V
        wid = W_LOGITS
        targets = uniform_targets(T, V, wid, self.seed)
        n_spike = int(round(self.spike_frac * T))
        spike_rows = np.zeros(T, dtype=bool)
        if n_spike:
            spike_rows[rng(wid, S_SPIKE, 0, self.seed).choice(T, size=n_spike, replace=False)] = True
        spike = np.float32(self.spike)

        def hook(r0, r1, blk):
            rows = np.nonzero(spike_rows[r0:r1])[0]
            blk[rows, targets[r0 + rows]] += spike

        logits = normal_bits((T, V), self.sigma, self.precision, wid, S_VALUES, self.seed, hook)
        mask = packed_response_mask(T, self.run_lo, self.run_hi, self.prompt_frac, wid, self.seed)
        self.arrays = dict(logits=logits, targets=targets, mask=mask, spike_rows=spike_rows)
        return self


@dataclass
class LMHead:
    """hidden bf16 [T, h] ~ N(0,1), W bf16 [V, h] ~ N(0, w_sigma^2), packed
    sequences with a prompt fraction unscored, uniform targets; optional
    upstream gradients g_lp ~ N(0,1), g_H ~ N(0, 0.1^2)."""
    T: int = 32768
    h: int = 5120
    V: int = 151936
    w_sigma: float = 0.02
    seq_lo: int = 512
    seq_hi: int = 8192
    prompt_frac: float = 0.30
    all_scored: bool = False
    temperature: float = 0.7
    tile_rows: int = 4096
    grads: bool = False
    g_H_sigma: float = 0.1
    workload: int = W_LM_HEAD_FWD
    seed: int = ROOT_SEED
    arrays: dict = field(default_factory=dict, repr=False)

    def build(self):
        wid = self.workload
        hidden = normal_bits((self.T, self.h), 1.0, "bf16", wid, S_VALUES, self.seed)
        weight = normal_bits((self.V, self.h), self.w_sigma, "bf16", wid, S_WEIGHT, self.seed)
        targets = uniform_targets(self.T, self.V, wid, self.seed)
        if self.all_scored:
            mask = np.ones(self.T, dtype=np.uint8)
        else:
            mask = packed_response_mask(self.T, self.seq_lo, self.seq_hi, self.prompt_frac, wid, self.seed)
        self.arrays = dict(hidden=hidden, weight=weight, targets=targets, mask=mask)
        if self.grads:
            self.arrays["grad_logprob"] = normal_f32(self.T, 1.0, wid, S_GRAD_LP, self.seed)
            self.arrays["grad_entropy"] = normal_f32(self.T, self.g_H_sigma, wid, S_GRAD_H, self.seed)
        return self


@dataclass
class KLPair:
    """student fp16 [T, V] ~ N(0, 4^2); teacher = fp16(student + N(0, 0.5^2));
    uniform targets; Bernoulli(0.6) diff mask."""
    T: int = 16384
    V: int = 129280
    sigma: float = 4.0
    noise: float = 0.5
    mask_p: float = 0.6
    precision: str = "fp16"
    seed: int = ROOT_SEED
    arrays: dict = field(default_factory=dict, repr=False)

    def build(self):
        T, V = self.T, self.V
        wid = W_KL
        student = normal_bits((T, V), self.sigma, self.precision, wid, S_VALUES, self.seed)
        to_f32 = _bits_to_f32_fn(self.precision)
        conv = f32_to_bf16_bits if self.precision == "bf16" else f32_to_fp16_bits
        teacher = np.empty_like(student)

        def fill(ib):
            i, (r0, r1) = ib
            g = rng(wid, S_NOISE, i, self.seed)
            n = g.standard_normal((r1 - r0, V), dtype=np.float32) * np.float32(self.noise)
            teacher[r0:r1] = conv(to_f32(student[r0:r1]) + n)

        blocks = list(enumerate(_row_blocks(T, V)))
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, blocks))
        targets = uniform_targets(T, V, wid, self.seed)
        diff_mask = bernoulli_mask(T, self.mask_p, wid, self.seed)
        self.arrays = dict(student=student, teacher=teacher, targets=targets, diff_mask=diff_mask)
        return self


def perturbed_bits(base: np.ndarray, precision: str, sigma: float, workload: int, stream: int,
                   seed: int = ROOT_SEED) -> np.ndarray:
    """round(base + N(0, sigma^2)) in `precision`, the noise drawn in fp32 per row block."""
    rows, cols = base.shape
    to_f32 = _bits_to_f32_fn(precision)
    conv = f32_to_bf16_bits if precision == "bf16" else f32_to_fp16_bits
    out = np.empty_like(base)

    def fill(ib):
        i, (r0, r1) = ib
        g = rng(workload, stream, i, seed)
        n = g.standard_normal((r1 - r0, cols), dtype=np.float32) * np.float32(sigma)
        out[r0:r1] = conv(to_f32(base[r0:r1]) + n)

    blocks = list(enumerate(_row_blocks(rows, cols)))
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, blocks))
    return out


@dataclass
class KLHeads:
    """Student and teacher last hidden states and output heads, bf16:
    student hidden [T, h] ~ N(0,1), student W [V, h] ~ N(0, w_sigma^2);
    teacher hidden = bf16(student hidden + N(0, h_noise^2)), teacher W =
    bf16(student W + N(0, w_noise^2)) (a teacher close to the student, as in
    distillation); all rows scored unless prompt_frac > 0; uniform targets;
    Bernoulli(0.6) diff mask; optional g_kl ~ N(0,1)."""
    T: int = 16384
    h: int = 7168
    V: int = 129280
    w_sigma: float = 0.02
    h_noise: float = 0.3
    w_noise: float = 0.005
    prompt_frac: float = 0.0
    mask_p: float = 0.6
    tile_rows: int = 4096
    grads: bool = False
    workload: int = W_KL_HEADS
    seed: int = ROOT_SEED
    arrays: dict = field(default_factory=dict, repr=False)

    def build(self):
        wid = self.workload
        hs = normal_bits((self.T, self.h), 1.0, "bf16", wid, S_VALUES, self.seed)
        ws = normal_bits((self.V, self.h), self.w_sigma, "bf16", wid, S_WEIGHT, self.seed)
        ht = perturbed_bits(hs, "bf16", self.h_noise, wid, S_NOISE, self.seed)
        wt = perturbed_bits(ws, "bf16", self.w_noise, wid, S_NOISE_W, self.seed)
        if self.prompt_frac > 0:
            mask = packed_response_mask(self.T, 512, 8192, self.prompt_frac, wid, self.seed)
        else:
            mask = np.ones(self.T, dtype=np.uint8)
        self.arrays = dict(student_hidden=hs, student_weight=ws, teacher_hidden=ht, teacher_weight=wt, mask=mask,
                           targets=uniform_targets(self.T, self.V, wid, self.seed),
                           diff_mask=bernoulli_mask(self.T, self.mask_p, wid, self.seed))
        if self.grads:
            self.arrays["grad_kl"] = normal_f32(self.T, 1.0, wid, S_GRAD_KL, self.seed)
        return self


def _bits_to_f32_fn(precision: str):
    if precision == "fp16":
        return lambda b: b.view(np.float16).astype(np.float32)
    return lambda b: (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def tiny_lm_head(seed: int = ROOT_SEED) -> LMHead:
    """T=64, h=256, V=1024, all rows scored, temperature 1.0, tile 16."""
    return LMHead(T=64, h=256, V=1024, all_scored=True, temperature=1.0, tile_rows=16,
                  workload=W_TINY_LM_HEAD, seed=seed).build()
