"""The binding loads liblp.so after PyTorch's own HIP runtime, whatever the
caller touches first: a fresh child process that loads the library before
using torch still computes the tiny fused forward correctly (with liblp.so
loaded first, a second HIP runtime came up and every launch failed with
"no device")."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
from entropy_chunked_row_amd import _lib
lib = _lib.load()                      # the library first ...
import numpy as np, torch              # ... torch afterwards
import entropy_chunked_row_amd as lp, synth
from oracle import lp_oracle as O
cfg = synth.tiny_lm_head(); A = cfg.arrays
dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
hid = dev(A["hidden"].view(np.int16)).view(torch.bfloat16); W = dev(A["weight"].view(np.int16)).view(torch.bfloat16)
lpv, H, _ = lp.lp_lm_head_logprobs_entropy(hid, W, dev(A["targets"]), dev(A["mask"]), cfg.temperature, cfg.tile_rows)
lp_o, H_o, _ = O.lm_head_logprobs_entropy(O.widen_bf16(A["hidden"]), O.widen_bf16(A["weight"]), A["targets"],
                                          A["mask"], cfg.temperature)
err = max(np.abs(lpv.cpu().numpy() - lp_o).max(), np.abs(H.cpu().numpy() - H_o).max())
print("max abs err", err)
sys.exit(0 if err <= 2e-3 else 3)
"""


def test_library_loaded_before_torch_in_a_fresh_process():
    p = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, (p.returncode, p.stdout[-2000:], p.stderr[-2000:])
