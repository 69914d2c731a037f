"""CPU checks of bench.py's host logic: the one-GPU contract, the source
hash that ties the committed PMC summary to the kernel sources, and the
board-power sampler."""
import os
import subprocess
import sys
import time

import pytest

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


def test_power_sampler_reads_hwmon(monkeypatch, tmp_path):
    (tmp_path / "power1_input").write_text("1234500000\n")
    (tmp_path / "power1_cap").write_text("1400000000\n")
    monkeypatch.setattr(bench, "_hwmon_dir", lambda: str(tmp_path))
    with bench._PowerSampler() as pw:
        time.sleep(0.05)
    s = pw.summary()
    assert s["samples"] >= 1 and s["mean_w"] == pytest.approx(1234.5) and s["max_w"] == pytest.approx(1234.5)
    assert s["cap_w"] == pytest.approx(1400.0)
    monkeypatch.setattr(bench, "_hwmon_dir", lambda: None)
    with bench._PowerSampler() as pw:
        pass
    assert pw.summary() is None
