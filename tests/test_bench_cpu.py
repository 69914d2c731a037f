"""CPU checks of bench.py's host logic: the one-GPU contract, and the source
hash that ties the committed PMC summary to the kernel sources."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_comment_stripping_keeps_code_and_strings():
    src = ('int a = 1; // tail\n/* block\ncomment */ const char* s = "x // y /* z */";\n'
           "char q = '\"'; char e = '\\\\'; int b;")
    out = bench._strip_comments(src)
    assert out == ('int a = 1; const char* s = "x // y /* z */"; char q = \'"\'; char e = \'\\\\\'; int b;')
    # comment and layout edits leave the stripped text, hence the hash, unchanged
    assert bench._strip_comments("int  a;\n// note\n  int b;") == bench._strip_comments("int a; int b; /* x */")
    assert bench._strip_comments("int a;") != bench._strip_comments("int b;")


def test_traffic_summary_parses():
    assert bench.measured_traffic("no_such_kernel") is None
    text = open(os.path.join(ROOT, "profiles", "hbm_traffic.md")).read()
    assert "```json" in text and "source_sha256" in text
