"""The no-alloc fused LM-head forward (static device scratch) against the
workspace form, through the C ABI: two calls in a row, the second with a
smaller input, each bitwise equal to the workspace form (same kernels, same
launch shapes) and within the fused tolerance of the fp64 oracle."""
import ctypes

import numpy as np
import pytest

import synth
from oracle import lp_oracle as O
from tests.helpers import host, max_abs_err, to_dev, to_dev_bits

pytestmark = pytest.mark.gpu
TOL_FWD = 2e-3


def _case(T, h, V, seed):
    rng = np.random.default_rng(seed)
    hid = synth.f32_to_bf16_bits(rng.normal(0, 1, size=(T, h)).astype(np.float32))
    W = synth.f32_to_bf16_bits(rng.normal(0, 0.05, size=(V, h)).astype(np.float32))
    y = rng.integers(0, V, size=T).astype(np.int64)
    m = (rng.random(T) < 0.7).astype(np.uint8)
    return hid, W, y, m


def _call_both(lib, torch, hid, W, y, m, tau, tile):
    T, h = hid.shape
    V = W.shape[0]
    hd, Wd, yd, md = to_dev_bits(hid, "bf16"), to_dev_bits(W, "bf16"), to_dev(y), to_dev(m)
    s = torch.cuda.current_stream().cuda_stream
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    outs = []
    for form in ("workspace", "noalloc"):
        lp = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
        H = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
        lse = torch.full((T,), 7.0, dtype=torch.float32, device="cuda")
        if form == "workspace":
            nb = lib.lp_lm_head_workspace_bytes(T, h, V, tile, 0)
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
            st = lib.lp_lm_head_logprobs_entropy(p(hd), h, p(Wd), h, T, h, V, p(yd), p(md), tau, tile, p(lp), p(H),
                                                 p(lse), p(ws), nb, s)
        else:
            assert lib.lp_lm_head_workspace_bytes(T, h, V, tile, 0) <= 64 << 20
            st = lib.lp_lm_head_logprobs_entropy_noalloc(p(hd), h, p(Wd), h, T, h, V, p(yd), p(md), tau, tile,
                                                         p(lp), p(H), p(lse), s)
        assert st == 0, lib.lp_last_error()
        torch.cuda.synchronize()
        outs.append([host(t) for t in (lp, H, lse)])
    return outs


def test_noalloc_forward_matches_workspace_form_on_two_calls():
    import torch

    import entropy_chunked_row_amd as lpm
    lib = lpm.load()
    # first call: direct-to-LDS tiles, several launches; second: a smaller input (generic tiles, h % 64 != 0)
    for T, h, V, tile, tau, seed in ((3000, 256, 20000, 256, 0.7, 1), (700, 72, 5003, 128, 1.3, 2)):
        hid, W, y, m = _case(T, h, V, seed)
        (lp_w, H_w, lse_w), (lp_n, H_n, lse_n) = _call_both(lib, torch, hid, W, y, m, tau, tile)
        assert np.array_equal(lp_w, lp_n) and np.array_equal(H_w, H_n) and np.array_equal(lse_w, lse_n), (T, h, V)
        lp_o, H_o, lse_o = O.lm_head_logprobs_entropy(O.widen_bf16(hid), O.widen_bf16(W), y, m, tau)
        assert max_abs_err(lp_n, lp_o) <= TOL_FWD and max_abs_err(H_n, H_o) <= TOL_FWD
        assert max_abs_err(lse_n, lse_o) <= TOL_FWD
        assert not lp_n[m == 0].any()


def test_noalloc_refuses_shapes_beyond_its_scratch():
    import entropy_chunked_row_amd as lpm
    lib = lpm.load()
    FAKE = 0x10000
    # the full forward workload at 4096-row tiles needs about 233 MB of scratch: refused before any launch
    st = lib.lp_lm_head_logprobs_entropy_noalloc(FAKE, 5120, FAKE, 5120, 32768, 5120, 151936, FAKE, None, 0.7, 4096,
                                                 FAKE, None, None, None)
    assert st == 3 and b"static scratch" in lib.lp_last_error()
