"""bench.py's one-line JSON contract, on a short run of the headline path and
the logits-input path (in-process: no child program is started from a
process that already uses the GPU)."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


def test_bench_prints_one_json_line_with_the_contract(monkeypatch, capsys):
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--paths", "lm_head_fwd,logits_input,tiny_lm_head", "--steps",
                                      "2", "--warmup", "1", "--settle-seconds", "0.2", "--cpu-seconds", "1",
                                      "--cpu-seconds-path", "0.5"])
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["dtype"] == "bf16" and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert isinstance(d["config"]["workload"], str) and "model" not in d["config"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    assert r["traffic"] is None or r["traffic"] > 0
    lg = r["library_gemm_same_shape"]
    assert lg["ms_per_call"] > 0 and r["frac_of_library_gemm_same_shape"] == pytest.approx(
        r["achieved"] / lg["achieved_tflops"])
    z = r["same_launch_on_zero_operands"]
    assert z["kernel_ms_per_step"] > 0 and 0 < z["frac"] < 1.2
    for pw in (r["board_power_during_timed_steps"], z["board_power"]):
        assert pw is None or (pw["samples"] >= 1 and 0 < pw["mean_w"] <= pw["max_w"] < 5000)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and isinstance(c["sample"], str)
    assert c["parity_max_abs_err"] <= c["parity_tol"]
    li = d["paths"]["logits_input"]["roofline"]
    assert li["bound"] == "hbm" and li["unit"] == "GB/s" and li["peak"] == 8000.0 and 0 < li["frac"] < 1.5
    # every path: the oracle timed beside it (with parity on its rows) and the memory one call allocates
    for name, path in [("lm_head_fwd", d)] + list(d["paths"].items()):
        c = path["cpu_baseline"]
        assert c["kind"] == "oracle" and c["value"] > 0 and c["parity_max_abs_err"] <= c["parity_tol"], name
        mem = path["memory"]
        assert mem["within_workspace_plus_outputs"], (name, mem)
        if name != "tiny_lm_head":  # 64 x 1024 logits are smaller than the workspace's fixed parts
            assert mem["peak_delta_bytes"] < 0.05 * mem["fp32_logits_bytes"], (name, mem)
    tiny = d["paths"]["tiny_lm_head"]
    assert tiny["roofline"] is None and tiny["us_per_call"] > 0
    # second denominators measured on this GPU: read probe, MFMA probe with its clock, library GEMM
    a = d["achievable"]
    assert a["hbm_read_gbs"] > 1000 and a["bf16_mfma_tflops"] > 500 and a["bf16_gemm_tflops"] > 100
    assert a["mfma_probe_sclk_mhz"] is None or 100 < a["mfma_probe_sclk_mhz"] < 5000
    # v_exp_f32: at most one per lane per clock on a SIMD of 16 lanes x 4 SIMDs, so below 64 per clock per CU
    assert a["exp2_per_s"] > 1e11 and (a["exp2_per_clk_per_cu"] is None or 1 < a["exp2_per_clk_per_cu"] <= 64.5)
    assert 0 < li["exp2_share_of_probe_rate"] < 1
    assert r["frac_of_achievable"] == pytest.approx(r["achieved"] / a["bf16_mfma_tflops"])
