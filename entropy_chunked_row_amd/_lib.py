"""ctypes view of liblp.so: symbol loading and C signatures only.

Loading the library does not touch the GPU (it imports torch first, whose HIP
runtime liblp.so then binds to).  There is no fallback: if the
library is missing the caller gets an error telling it to build.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblp.so")

c_i64 = ctypes.c_int64
c_vp = ctypes.c_void_p
c_f = ctypes.c_float
c_int = ctypes.c_int

# name -> (restype, argtypes); mirrors include/lp.h
SIGNATURES = {
    "lp_version": (c_int, []),
    "lp_status_string": (ctypes.c_char_p, [c_int]),
    "lp_last_error": (ctypes.c_char_p, []),
    "lp_logprobs_entropy": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_f, c_i64, c_vp, c_vp, c_vp]),
    "lp_lm_head_workspace_bytes": (ctypes.c_size_t, [c_i64, c_i64, c_i64, c_i64, c_int]),
    "lp_lm_head_fast_tiles": (c_int, [c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_int]),
    "lp_lm_head_logprobs_entropy": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_f, c_i64,
                                            c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "lp_lm_head_logprobs_entropy_noalloc": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp,
                                                    c_f, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "lp_lm_head_logprobs_entropy_backward": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_f,
                                                     c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                     ctypes.c_size_t, c_vp]),
    "lp_kl_full_vocab": (c_int, [c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                 c_vp]),
    "lp_prob_diff": (c_int, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp]),
    "lp_logprobs_entropy_k": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_f, c_i64, c_vp, c_vp,
                                      c_vp]),
    "lp_lm_head_logprobs_entropy_k": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_f,
                                              c_i64, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "lp_lm_head_logprobs_entropy_backward_k": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_i64,
                                                       c_vp, c_f, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                       ctypes.c_size_t, c_vp]),
    "lp_prob_diff_stats_workspace_bytes": (ctypes.c_size_t, []),
    "lp_prob_diff_stats": (c_int, [c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "lp_lm_head_kl_workspace_bytes": (ctypes.c_size_t, [c_i64, c_i64, c_i64, c_i64, c_int]),
    "lp_lm_head_kl": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64,
                              c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t,
                              c_vp]),
    "lp_lm_head_kl_backward": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64,
                                       c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t,
                                       c_vp]),
    "lp_timing_enable": (None, [c_int]),
    "lp_timing_read": (c_int, [ctypes.c_char_p, ctypes.POINTER(c_i64), ctypes.POINTER(ctypes.c_double)]),
    "lp_timing_clock": (c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64)]),
}

LP_OK, LP_ERR_INVALID_ARGUMENT, LP_ERR_UNSUPPORTED, LP_ERR_WORKSPACE_TOO_SMALL, LP_ERR_HIP = range(5)
LP_BF16, LP_FP16, LP_FP32 = range(3)

_lib = None


class LPError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {detail}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m entropy_chunked_row_amd.build` "
                           "(there is no CPU fallback)")
    # PyTorch ships its own HIP runtime.  Loaded first, it is the runtime
    # liblp.so binds to (same soname); loaded after liblp.so, a second copy of
    # the runtime would come up beside the one liblp.so brought in, and one of
    # the two then sees no device.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the binding needs torch for tensors anyway
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != LP_OK:
        lib = load()
        raise LPError(fn, status, lib.lp_last_error().decode(errors="replace"))
