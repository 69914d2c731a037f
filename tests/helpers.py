"""Shared test utilities: moving synthetic bit arrays to the GPU, comparisons."""
import numpy as np


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev_bits(bits: np.ndarray, dtype: str):
    """uint16 bit array -> device tensor of bf16/fp16 with the same bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev())
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def max_abs_err(got, want, rows=None):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if rows is not None:
        got, want = got[rows], want[rows]
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - want)))


def grad_errors(got, want):
    """(relative Frobenius error, max|diff| / max|want|)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    nrm = np.linalg.norm(want)
    mx = np.max(np.abs(want)) if want.size else 0.0
    fro = np.linalg.norm(got - want) / nrm if nrm > 0 else np.linalg.norm(got)
    mad = np.max(np.abs(got - want)) / mx if mx > 0 else np.max(np.abs(got)) if got.size else 0.0
    return float(fro), float(mad)


def oracle_by_row_blocks(fn, rows, block=128, workers=None):
    """fn(rows_subset) -> tuple of per-row arrays, evaluated over blocks of
    `rows` in a thread pool (numpy releases the GIL inside its kernels) and
    concatenated in row order.  For full-size parity on every scored row."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    rows = np.asarray(rows)
    if workers is None:
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
    parts = [rows[i:i + block] for i in range(0, len(rows), block)]
    with ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(fn, parts))
    return tuple(np.concatenate([o[k] for o in outs]) for k in range(len(outs[0])))
