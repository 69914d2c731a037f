"""Memory audit: the library allocates no device memory (scratch comes from
the caller's workspace), and the workspace of the fused paths stays below
one [rows x vocab] fp32 buffer at the benchmark shapes (the KL forward holds
one chunk of the teacher's logits)."""
import numpy as np
import pytest

import synth
from tests.helpers import to_dev, to_dev_bits

pytestmark = pytest.mark.gpu


def _free_bytes(torch):
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def test_entry_points_allocate_no_device_memory():
    import torch
    from entropy_chunked_row_amd import _lib
    lib = _lib.load()
    rng = np.random.default_rng(4)
    T, h, V, tile = 300, 128, 5000, 128
    hid = to_dev_bits(synth.f32_to_bf16_bits(rng.normal(0, 1, (T, h)).astype(np.float32)), "bf16")
    W = to_dev_bits(synth.f32_to_bf16_bits(rng.normal(0, 0.05, (V, h)).astype(np.float32)), "bf16")
    logits = to_dev_bits(synth.f32_to_bf16_bits(rng.normal(0, 3, (T, V)).astype(np.float32)), "bf16")
    y = to_dev(rng.integers(0, V, T).astype(np.int64))
    m = to_dev((rng.random(T) < 0.7).astype(np.uint8))
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = [torch.empty(T, **f32) for _ in range(6)]
    g = torch.randn(T, **f32)
    dH = torch.empty((T, h), **f32)
    dW = torch.empty((V, h), **f32)
    ws = torch.empty(max(lib.lp_lm_head_workspace_bytes(T, h, V, tile, 1),
                         lib.lp_lm_head_kl_workspace_bytes(T, h, V, tile, 1)), dtype=torch.uint8, device="cuda")
    stats = torch.empty(5, dtype=torch.float64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()
    n = ws.numel()

    calls = {
        "lp_logprobs_entropy": lambda: lib.lp_logprobs_entropy(p(logits), 0, T, V, V, p(y), p(m), 0.7, 64,
                                                               p(outs[0]), p(outs[1]), s),
        "lp_lm_head_logprobs_entropy": lambda: lib.lp_lm_head_logprobs_entropy(
            p(hid), h, p(W), h, T, h, V, p(y), p(m), 0.7, tile, p(outs[0]), p(outs[1]), p(outs[2]), p(ws), n, s),
        "lp_lm_head_logprobs_entropy_backward": lambda: lib.lp_lm_head_logprobs_entropy_backward(
            p(hid), h, p(W), h, T, h, V, p(y), p(m), 0.7, tile, p(outs[2]), p(outs[1]), p(g), p(g), p(dH), p(dW),
            p(ws), n, s),
        "lp_kl_full_vocab": lambda: lib.lp_kl_full_vocab(p(logits), p(logits), 0, T, V, V, V, p(outs[0]), p(y),
                                                         p(m), p(outs[1]), p(outs[2]), p(outs[3]), s),
        "lp_lm_head_kl": lambda: lib.lp_lm_head_kl(p(hid), h, p(W), h, h, p(hid), h, p(W), h, h, T, V, p(m), p(y),
                                                   None, tile, *[p(o) for o in outs], p(ws), n, s),
        "lp_lm_head_kl_backward": lambda: lib.lp_lm_head_kl_backward(
            p(hid), h, p(W), h, h, p(hid), h, p(W), h, h, T, V, p(m), tile, p(outs[4]), p(outs[5]), p(g), p(dH),
            p(dW), p(ws), n, s),
        "lp_prob_diff_stats": lambda: lib.lp_prob_diff_stats(p(outs[0]), p(outs[1]), p(m), T, p(stats), p(ws), n, s),
    }
    for name, call in calls.items():
        assert call() == 0, (name, lib.lp_last_error())  # warm-up: code objects load on first use
    for name, call in calls.items():
        before = _free_bytes(torch)
        for _ in range(3):
            assert call() == 0, (name, lib.lp_last_error())
        after = _free_bytes(torch)
        assert after == before, (name, before - after)


def test_workspace_far_below_a_logits_buffer():
    from entropy_chunked_row_amd import _lib
    lib = _lib.load()
    # fused forward (32768 rows, h 5120, V 151936, tile 4096) and forward + backward (114688 rows)
    fw = lib.lp_lm_head_workspace_bytes(32768, 5120, 151936, 4096, 0)
    bw = lib.lp_lm_head_workspace_bytes(114688, 5120, 151936, 4096, 1)
    kl = lib.lp_lm_head_kl_workspace_bytes(16384, 7168, 129280, 4096, 0)
    assert fw < 32768 * 151936 * 4 / 50  # partial states of up to 8 tiles of 4096 rows
    assert bw < 114688 * 151936 * 4 / 10
    assert kl < 16384 * 129280 * 4 / 3  # one 4096-row chunk of the teacher's fp32 logits, no [T x V]


def test_no_rows_through_the_c_abi():
    """T = 0 (and n = 0): every entry point returns OK; a backward still
    defines the weight gradient of an empty sum, so a requested dW is
    overwritten with zeros; the aggregates of no position are count 0 and a
    NaN Pearson."""
    import math
    import torch
    from entropy_chunked_row_amd import _lib
    lib = _lib.load()
    h, V, K, tile = 64, 300, 2, 16
    dev = "cuda"
    bf = lambda *shape: torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    f32 = lambda *shape: torch.zeros(shape, dtype=torch.float32, device=dev)
    hid, W = bf(1, h), bf(V, h)
    y = torch.zeros(K, dtype=torch.int64, device=dev)
    m = torch.ones(1, dtype=torch.uint8, device=dev)
    outs = [f32(K) for _ in range(6)]
    dH = f32(1, h)
    s = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    n = ws.numel()

    def dw_sentinel():
        return torch.full((V, h), 7.0, dtype=torch.float32, device=dev)

    assert lib.lp_lm_head_logprobs_entropy(p(hid), h, p(W), h, 0, h, V, p(y), p(m), 0.7, tile, p(outs[0]), p(outs[1]),
                                           p(outs[2]), p(ws), n, s) == 0
    assert lib.lp_lm_head_logprobs_entropy_k(p(hid), h, p(W), h, 0, h, V, p(y), K, p(m), 0.7, tile, p(outs[0]),
                                             p(outs[1]), p(outs[2]), p(ws), n, s) == 0
    assert lib.lp_logprobs_entropy_k(p(W), 0, 0, V, V, p(y), K, p(m), 0.7, 4, p(outs[0]), p(outs[1]), s) == 0
    assert lib.lp_lm_head_kl(p(hid), h, p(W), h, h, p(hid), h, p(W), h, h, 0, V, p(m), p(y), p(m), tile,
                             *[p(o) for o in outs], p(ws), n, s) == 0
    dW = dw_sentinel()
    assert lib.lp_lm_head_logprobs_entropy_backward(p(hid), h, p(W), h, 0, h, V, p(y), p(m), 0.7, tile, p(outs[2]),
                                                    p(outs[1]), p(outs[0]), p(outs[3]), p(dH), p(dW), p(ws), n, s) == 0
    torch.cuda.synchronize()
    assert not dW.any()
    dW = dw_sentinel()
    assert lib.lp_lm_head_logprobs_entropy_backward_k(p(hid), h, p(W), h, 0, h, V, p(y), K, p(m), 0.7, tile,
                                                      p(outs[2]), p(outs[1]), p(outs[0]), p(outs[3]), p(dH), p(dW),
                                                      p(ws), n, s) == 0
    torch.cuda.synchronize()
    assert not dW.any()
    dW = dw_sentinel()
    assert lib.lp_lm_head_kl_backward(p(hid), h, p(W), h, h, p(hid), h, p(W), h, h, 0, V, p(m), tile, p(outs[4]),
                                      p(outs[5]), p(outs[0]), p(dH), p(dW), p(ws), n, s) == 0
    torch.cuda.synchronize()
    assert not dW.any()
    stats = torch.full((5,), 7.0, dtype=torch.float64, device=dev)
    assert lib.lp_prob_diff_stats(p(outs[0]), p(outs[1]), None, 0, p(stats), p(ws), n, s) == 0
    got = stats.cpu().tolist()
    assert got[:4] == [0.0, 0.0, 0.0, 0.0] and math.isnan(got[4])
