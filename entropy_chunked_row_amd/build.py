"""Builds liblp.so (the C-ABI library) in-tree for gfx950 with hipcc.

    python -m entropy_chunked_row_amd.build

Objects go to <repo>/_build/, the library to entropy_chunked_row_amd/liblp.so;
the bench-only read probe to entropy_chunked_row_amd/liblp_probe.so.
Every call recompiles (it is also the "does it build" check).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "liblp.so")
SOURCES = ["lp_api.hip", "lp_rows.hip", "lp_lmhead.hip", "lp_timing.hip"]
# measurement helper for bench.py (HBM read probe), a library of its own
PROBE_SRC = os.path.join(PKG, "probe", "lp_probe.hip")
PROBE_OUT = os.path.join(PKG, "liblp_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 VALU ops anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build liblp.so)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops' is not a recognized feature" not in ln]
    if p.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[cc, *HIPCC_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    probe_tmp = PROBE_OUT + ".tmp"
    cmds.append([cc, *HIPCC_FLAGS, "-shared", "-I", INCLUDE, PROBE_SRC, "-o", probe_tmp])
    with ThreadPoolExecutor(len(cmds)) as ex:
        logs = list(ex.map(_run, cmds))
    os.replace(probe_tmp, PROBE_OUT)
    tmp = OUT + ".tmp"
    logs.append(_run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, OUT)
    if verbose:
        for lg in logs:
            if lg.strip():
                print(lg)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
