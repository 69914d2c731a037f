#!/usr/bin/env python3
"""Benchmark of the per-token log-prob / entropy hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--paths all|lm_head_fwd,...]

Headline (`value`): scored tokens/s of the fused LM-head forward (log-prob +
entropy of softmax(hidden @ W^T / 0.7)) on T = 32768 packed rows (about 70 %
scored), h = 5120, V = 151936, bf16, tile 4096 rows.  One step is one call of
lp_lm_head_logprobs_entropy with inputs already resident in HBM.  The same
JSON line carries the other paths measured the same way (the tiny fused head
in absolute microseconds, logits-input rows, exact KL + prob diff, fused
forward + backward, KL through both heads), each with the roofline of its
dominant kernels from live per-launch HIP-event timing, the fp64 oracle timed
on the host cores over a bounded sample of the same workload (and compared
with the GPU's outputs on those rows), and the device memory one call
allocates.  Each path runs its step untimed for --settle-seconds (steady GPU
clocks after the host-side input generation), then W warm-up steps, then
exactly K timed steps.  The board power (amdgpu hwmon, sampled on a host
thread) is recorded over each timed region; the forward also records the
shader clock its workgroups ran at and repeats its launch on all-zero
operands, which shows how much of the gap to the datasheet rate is the power
limit rather than the kernel.

Inputs are seeded and synthetic (see synth/).  The fp64 oracle is used only in
the CPU-baseline legs; every path's parity at full size is in tests/.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scored tokens/s, fused LM-head logprob+entropy; % of MFMA / HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
ALL_PATHS = ("lm_head_fwd", "tiny_lm_head", "logits_input", "kl_prob_diff", "lm_head_fwd_bwd", "kl_lm_head")
MFMA_FLOP = 2 * 32 * 32 * 16   # one v_mfma_f32_32x32x16_bf16


def to_dev_bits(bits, dtype):
    """uint16 bit array -> device bf16/fp16 tensor with the same bits."""
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def to_dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _strip_comments(text):
    """C++ source without comments and with whitespace runs collapsed: two
    sources hash alike when they differ only in comments or layout."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def _csrc_sha256():
    """Hash of the kernel sources (comments and layout ignored) that the PMC
    summary in profiles/ must match."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "entropy_chunked_row_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_strip_comments(fh.read()).encode())
    return h.hexdigest()


def _pmc_doc():
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    try:
        text = open(path).read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        doc = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None
    if doc.get("source_sha256") != _csrc_sha256():
        return None
    return doc


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` (a timing name) from the committed PMC
    summary, or None when the kernel sources changed since the counters were
    taken."""
    doc = _pmc_doc()
    if doc is None:
        return None
    k = doc.get("kernels", {}).get(kernel)
    return None if k is None else k["bytes_per_launch"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _events_ms(torch, fn, steps):
    s = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(s)
    for _ in range(steps):
        fn()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


SETTLE_SECONDS = 2.0  # set from --settle-seconds in main()


def _hwmon_dir():
    """The amdgpu hwmon directory of the one visible GPU (board power in
    microwatts: power1_input, cap power1_cap), or None where sysfs shows none
    or several."""
    import glob
    found = sorted(d for d in glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")
                   if os.path.exists(os.path.join(d, "power1_input")))
    return found[0] if len(found) == 1 else None


class _PowerSampler:
    """Samples the board power every 10 ms on a host thread while a timed
    region runs (reads sysfs only; nothing on the GPU)."""

    def __init__(self):
        self.dir = _hwmon_dir()
        self.samples = []

    def _read(self, name):
        try:
            with open(os.path.join(self.dir, name)) as f:
                return int(f.read()) / 1e6
        except (OSError, ValueError, TypeError):
            return None

    def __enter__(self):
        import threading
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                w = self._read("power1_input")
                if w is not None:
                    self.samples.append(w)
                self._stop.wait(0.01)

        self._t = threading.Thread(target=run, daemon=True)
        if self.dir:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.dir:
            self._t.join()

    def summary(self):
        if not self.samples:
            return None
        return dict(mean_w=sum(self.samples) / len(self.samples), max_w=max(self.samples),
                    samples=len(self.samples), cap_w=self._read("power1_cap"))


def _timed(lp, torch, fn, steps, warmup, kernels, clocks=False):
    # Clock settle: the GPU idles while a path's inputs are generated on the
    # host, and it needs some time under load to reach its steady clocks.  Run
    # the step untimed for SETTLE_SECONDS first, then the W warm-up steps,
    # then exactly K timed steps.
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_SECONDS:
        fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    lp.lp_timing_enable(2 if clocks else True)
    with _PowerSampler() as pw:
        ms = _events_ms(torch, fn, steps)
    per_kernel = {k: lp.lp_timing_read(k) for k in kernels}
    per_kernel["_power"] = pw.summary()
    if clocks:
        per_kernel["_clock"] = lp.lp_timing_clock("k_fwd_tile")
    lp.lp_timing_enable(False)
    return ms, per_kernel


def _memory_audit(torch, call, workspace_bytes, output_bytes, fp32_logits_bytes):
    """Device memory one call allocates: the peak of torch's allocated bytes
    across the call (its outputs and, here, its workspace, both allocated by
    the binding) against workspace + outputs, and against the [T x V] fp32
    logits the method never forms."""
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    out = call()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    del out
    bound = workspace_bytes + output_bytes
    return dict(peak_delta_bytes=int(peak), workspace_bytes=int(workspace_bytes), output_bytes=int(output_bytes),
                within_workspace_plus_outputs=bool(peak <= bound + (1 << 20)),
                fp32_logits_bytes=int(fp32_logits_bytes), frac_of_fp32_logits=peak / fp32_logits_bytes)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover
        return 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _sample_rows(np, rows, n):
    """n rows spread over `rows` (seeded, sorted)."""
    if n >= len(rows):
        return np.asarray(rows)
    return np.sort(np.random.default_rng(20261202).choice(rows, n, replace=False))


def _oracle_timed(np, run, rows, seconds, n0):
    """Times run(sample) on growing samples of `rows` until one takes at least
    0.6 x `seconds` (or covers every row); returns (sample, seconds, result)."""
    n = min(n0, len(rows))
    while True:
        sample = _sample_rows(np, rows, n)
        t0 = time.perf_counter()
        res = run(sample)
        t = time.perf_counter() - t0
        if t >= 0.6 * seconds or n >= len(rows):
            return sample, t, res
        n = min(len(rows), int(n * min(8.0, max(2.0, seconds / max(t, 1e-3)))))


def _baseline(n, t, unit, sample, parity_err, parity_tol, **extra):
    d = dict(value=n / t, unit=unit, cores=_blas_threads(), kind="oracle", sample=sample, seconds=t,
             cpu_model=_cpu_model(), parity_rows=int(n), parity_max_abs_err=float(parity_err),
             parity_tol=parity_tol)
    d.update(extra)
    return d


class _LazyWeight:
    """Widens bf16 weight rows to fp64 only for the vocab block asked for."""

    def __init__(self, O, bits):
        self.O, self.bits, self.shape = O, bits, bits.shape

    def __getitem__(self, sl):
        return self.O.widen_bf16(self.bits[sl])


# ---------------------------------------------------------------------------
# paths
# ---------------------------------------------------------------------------

def bench_lm_head_fwd(lp, torch, np, synth, steps, warmup, cpu_seconds, cfg=None, tiny=False):
    cfg = cfg or synth.LMHead().build()
    A = cfg.arrays
    hid, W = to_dev_bits(A["hidden"], "bf16"), to_dev_bits(A["weight"], "bf16")
    y, m = to_dev(A["targets"]), to_dev(A["mask"])
    Ts = int(A["mask"].sum())
    ws_bytes = lp.lp_lm_head_workspace_bytes(cfg.T, cfg.h, cfg.V, cfg.tile_rows, False)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = {}

    def step():
        out["r"] = lp.lp_lm_head_logprobs_entropy(hid, W, y, m, cfg.temperature, cfg.tile_rows, workspace=ws)

    ms, kt = _timed(lp, torch, step, steps, warmup, ["k_fwd_tile", "k_fwd_merge", "k_compact"], clocks=not tiny)
    sclk, sclk_n = kt.pop("_clock", (None, 0))
    power = kt.pop("_power", None)
    flop_step = 2.0 * Ts * cfg.V * cfg.h
    n_launch, gemm_ms = kt["k_fwd_tile"]
    n_tiles = (Ts + cfg.tile_rows - 1) // cfg.tile_rows
    achieved = flop_step * steps / (gemm_ms * 1e-3) / 1e12
    rows_desc = f"T={cfg.T} rows, all scored" if tiny else f"T={cfg.T} packed rows ({Ts} scored)"
    wl = (f"{'tiny ' if tiny else ''}fused LM-head forward: {rows_desc}, h={cfg.h}, V={cfg.V}, bf16, "
          f"tau {cfg.temperature}, tile {cfg.tile_rows}")
    res = dict(workload=wl, T=cfg.T, scored_rows=Ts, h=cfg.h, V=cfg.V, temperature=cfg.temperature,
               tile_rows=cfg.tile_rows, ms_per_step=ms / steps, tokens_per_s=Ts * steps / (ms * 1e-3),
               kernel_ms_per_step={k: v[1] / steps for k, v in kt.items()})
    if tiny:
        # launch-bound: three launches of a few microseconds, no roofline claim; the call time is taken again
        # without the per-kernel events, which add their own few microseconds per launch
        plain_ms = _events_ms(torch, step, steps)
        res["ms_per_step"] = plain_ms / steps
        res["tokens_per_s"] = Ts * steps / (plain_ms * 1e-3)
        res["us_per_call"] = 1e3 * plain_ms / steps
        res["kernel_us_per_call"] = {k: 1e3 * v[1] / steps for k, v in kt.items()}
        res["roofline"] = None
    else:
        res["roofline"] = dict(
            bound="mfma", kernel="k_fwd_tile", kernel_ms_per_launch=gemm_ms / n_launch, achieved=achieved,
            peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=achieved / BF16_PEAK_TFLOPS,
            traffic=measured_traffic("k_fwd_tile"),
            traffic_unit="HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            algorithmic_hbm_bytes_per_launch=(n_tiles * cfg.V * cfg.h * 2 + Ts * cfg.h * 2) / (n_launch / steps),
            launches_per_step=n_launch / steps, kernel_ms_per_step=gemm_ms / steps,
            algorithmic_flop_per_step=flop_step, algorithmic_flop_per_launch=flop_step / (n_launch / steps),
            # the shader clock the kernel's workgroups ran at (last timed launch), and the fraction of the
            # datasheet rate scaled to that clock (the datasheet figure assumes 2.4 GHz)
            sclk_mhz_during_kernel=sclk or None, sclk_samples=sclk_n,
            frac_at_observed_clock=(achieved / (BF16_PEAK_TFLOPS * sclk / 2400.0)) if sclk else None,
            board_power_during_timed_steps=power,
            same_launch_on_zero_operands=_zero_operand_run(lp, torch, cfg, y, m, ws, flop_step),
            library_gemm_same_shape=_library_gemm_same_shape(torch, hid, W, m, flop_step))
        lib = res["roofline"]["library_gemm_same_shape"]
        res["roofline"]["frac_of_library_gemm_same_shape"] = achieved / lib["achieved_tflops"]
    res["memory"] = _memory_audit(
        torch, lambda: lp.lp_lm_head_logprobs_entropy(hid, W, y, m, cfg.temperature, cfg.tile_rows),
        ws_bytes, 3 * 4 * cfg.T, 4 * cfg.T * cfg.V)
    if cpu_seconds > 0:
        lpv, Hv, lsev = (t.cpu().numpy() for t in out["r"])
        from oracle import lp_oracle as O  # CPU-baseline leg only
        Wl = _LazyWeight(O, A["weight"])

        def run(rows):
            return O.lm_head_logprobs_entropy(O.widen_bf16(A["hidden"][rows]), Wl, A["targets"][rows], None,
                                              cfg.temperature)

        rows, t, (lp_o, H_o, lse_o) = _oracle_timed(np, run, np.nonzero(A["mask"])[0], cpu_seconds, 8)
        err = max(np.abs(lpv[rows] - lp_o).max(), np.abs(Hv[rows] - H_o).max(), np.abs(lsev[rows] - lse_o).max())
        res["cpu_baseline"] = _baseline(
            len(rows), t, "scored tokens/s",
            f"{len(rows)} scored rows of the same workload through the fp64 oracle (full V={cfg.V}, h={cfg.h})",
            err, 2e-3)
    del hid, W, y, m, ws, out
    torch.cuda.empty_cache()
    return res


def _zero_operand_run(lp, torch, cfg, y, m, ws, flop_step, steps=3):
    """The same forward launch on all-zero hidden rows and weights: identical
    instructions, loads and LDS traffic, but matrix-core inputs that never
    toggle.  Its clock and board power, next to the timed run's, show how far
    the timed run's clock is set by the board's power limit (context only; the
    reported throughput is the timed run on the seeded operands)."""
    hid0 = torch.zeros((cfg.T, cfg.h), dtype=torch.bfloat16, device="cuda")
    W0 = torch.zeros((cfg.V, cfg.h), dtype=torch.bfloat16, device="cuda")

    def step():
        lp.lp_lm_head_logprobs_entropy(hid0, W0, y, m, cfg.temperature, cfg.tile_rows, workspace=ws)

    ms, kt = _timed(lp, torch, step, steps, 1, ["k_fwd_tile"], clocks=True)
    sclk, n = kt["_clock"]
    gemm_ms = kt["k_fwd_tile"][1]
    del hid0, W0
    achieved = flop_step * steps / (gemm_ms * 1e-3) / 1e12
    return dict(kernel_ms_per_step=gemm_ms / steps, achieved_tflops=achieved, frac=achieved / BF16_PEAK_TFLOPS,
                sclk_mhz_during_kernel=sclk or None, board_power=kt["_power"])


def _library_gemm_same_shape(torch, hid, W, m, flop_step, steps=5):
    """Context only: the library bf16 GEMM (torch.matmul) of the scored hidden
    rows by the weight, bf16 logits out, on the forward workload's shape -- the
    matrix product alone, without the log-softmax / entropy the fused kernel
    folds in, and with the [rows x V] logits it writes."""
    hs = hid[torch.nonzero(m).flatten()].contiguous()
    out = torch.empty((hs.shape[0], W.shape[0]), dtype=torch.bfloat16, device="cuda")
    wt = W.t()

    def step():
        torch.matmul(hs, wt, out=out)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_SECONDS:
        step()
        torch.cuda.synchronize()
    with _PowerSampler() as pw:
        ms = _events_ms(torch, step, steps) / steps
    del hs, out
    achieved = flop_step / (ms * 1e-3) / 1e12
    return dict(ms_per_call=ms, achieved_tflops=achieved, frac=achieved / BF16_PEAK_TFLOPS, board_power=pw.summary(),
                op="torch.matmul(hidden[scored rows], weight^T), bf16 in and out")


def bench_tiny_lm_head(lp, torch, np, synth, steps, warmup, cpu_seconds):
    """T=64, h=256, V=1024, tile 16: launch-bound, reported in microseconds."""
    return bench_lm_head_fwd(lp, torch, np, synth, max(steps, 100), max(warmup, 10), cpu_seconds,
                             cfg=synth.tiny_lm_head(), tiny=True)


def bench_logits_input(lp, torch, np, synth, steps, warmup, cpu_seconds):
    cfg = synth.LogitsInput().build()
    A = cfg.arrays
    x, y, m = to_dev_bits(A["logits"], "bf16"), to_dev(A["targets"]), to_dev(A["mask"])
    Ts = int(A["mask"].sum())
    lpo = torch.empty(cfg.T, device="cuda")
    Ho = torch.empty(cfg.T, device="cuda")

    def step():
        lp.lp_logprobs_entropy(x, y, m, cfg.temperature, cfg.chunk_rows, logprob=lpo, entropy=Ho)

    ms, kt = _timed(lp, torch, step, steps, warmup, ["k_logprobs_entropy"])
    power = kt.pop("_power")
    n_launch, kms = kt["k_logprobs_entropy"]
    bytes_step = Ts * (2 * cfg.V + 8 + 8) + cfg.T * 1 + (cfg.T - Ts) * 8
    achieved = bytes_step * steps / (kms * 1e-3) / 1e9
    res = dict(
        workload=f"logits input: bf16 [{cfg.T}, {cfg.V}] ({Ts} scored rows), tau {cfg.temperature}, "
                 f"chunk {cfg.chunk_rows}",
        ms_per_step=ms / steps, tokens_per_s=Ts * steps / (ms * 1e-3),
        roofline=dict(bound="hbm", kernel="k_logprobs_entropy", kernel_ms_per_launch=kms / n_launch,
                      achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=measured_traffic("k_logprobs_entropy"),
                      traffic_unit="HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                      algorithmic_bytes_per_launch=bytes_step / (n_launch / steps),
                      launches_per_step=n_launch / steps, algorithmic_bytes_per_step=bytes_step,
                      board_power_during_timed_steps=power))
    res["memory"] = _memory_audit(torch, lambda: lp.lp_logprobs_entropy(x, y, m, cfg.temperature, cfg.chunk_rows),
                                  0, 2 * 4 * cfg.T, 4 * cfg.T * cfg.V)
    if cpu_seconds > 0:
        from oracle import lp_oracle as O  # CPU-baseline leg only
        lpv, Hv = lpo.cpu().numpy(), Ho.cpu().numpy()

        def run(rows):
            return O.logprobs_entropy(O.widen_bf16(A["logits"][rows]), A["targets"][rows], None, cfg.temperature)

        rows, t, (lp_o, H_o, _) = _oracle_timed(np, run, np.nonzero(A["mask"])[0], cpu_seconds, 64)
        err = max(np.abs(lpv[rows] - lp_o).max(), np.abs(Hv[rows] - H_o).max())
        res["cpu_baseline"] = _baseline(len(rows), t, "scored tokens/s",
                                        f"{len(rows)} scored rows of the same logits through the fp64 oracle", err,
                                        1e-5)
    del x, y, m, lpo, Ho
    torch.cuda.empty_cache()
    return res


def bench_kl(lp, torch, np, synth, steps, warmup, cpu_seconds):
    cfg = synth.KLPair().build()
    A = cfg.arrays
    u, v = to_dev_bits(A["student"], "fp16"), to_dev_bits(A["teacher"], "fp16")
    y, dm = to_dev(A["targets"]), to_dev(A["diff_mask"])
    out = {}

    def step():
        out["r"] = lp.lp_kl_full_vocab(u, v, y, dm)

    ms, kt = _timed(lp, torch, step, steps, warmup, ["k_kl_full_vocab"])
    power = kt.pop("_power")
    n_launch, kms = kt["k_kl_full_vocab"]
    bytes_step = cfg.T * (2 * 2 * cfg.V + 8 + 1 + 4 * 4)
    achieved = bytes_step * steps / (kms * 1e-3) / 1e9
    res = dict(
        workload=f"exact KL(teacher||student) + target log-probs + masked prob diff: fp16 [{cfg.T}, {cfg.V}] x 2",
        ms_per_step=ms / steps, tokens_per_s=cfg.T * steps / (ms * 1e-3),
        roofline=dict(bound="hbm", kernel="k_kl_full_vocab", kernel_ms_per_launch=kms / n_launch,
                      achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=measured_traffic("k_kl_full_vocab"),
                      traffic_unit="HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                      algorithmic_bytes_per_launch=bytes_step / (n_launch / steps),
                      launches_per_step=n_launch / steps, algorithmic_bytes_per_step=bytes_step,
                      board_power_during_timed_steps=power))
    res["memory"] = _memory_audit(torch, lambda: lp.lp_kl_full_vocab(u, v, y, dm), 0, 4 * 4 * cfg.T,
                                  2 * 4 * cfg.T * cfg.V)
    if cpu_seconds > 0:
        from oracle import lp_oracle as O  # CPU-baseline leg only
        got = [t.cpu().numpy() for t in out["r"]]

        def run(rows):
            return O.kl_and_prob_diff(O.widen_fp16(A["student"][rows]), O.widen_fp16(A["teacher"][rows]),
                                      A["targets"][rows], A["diff_mask"][rows])

        rows, t, want = _oracle_timed(np, run, np.arange(cfg.T), cpu_seconds, 32)
        err = max(np.abs(g[rows] - w).max() for g, w in zip(got, want))
        res["cpu_baseline"] = _baseline(len(rows), t, "tokens/s",
                                        f"{len(rows)} rows of both models' logits through the fp64 oracle "
                                        "(KL, both target log-probs, masked diff)", err, 1e-5)
    del u, v, y, dm, out
    torch.cuda.empty_cache()
    return res


def bench_lm_head_fwd_bwd(lp, torch, np, synth, steps, warmup, cpu_seconds):
    cfg = synth.LMHead(T=114688, prompt_frac=0.2, temperature=1.0, grads=True, workload=synth.W_LM_HEAD_BWD).build()
    A = cfg.arrays
    hid, W = to_dev_bits(A["hidden"], "bf16"), to_dev_bits(A["weight"], "bf16")
    y, m = to_dev(A["targets"]), to_dev(A["mask"])
    glp, gH = to_dev(A["grad_logprob"]), to_dev(A["grad_entropy"])
    Ts = int(A["mask"].sum())
    wsf_bytes = lp.lp_lm_head_workspace_bytes(cfg.T, cfg.h, cfg.V, cfg.tile_rows, False)
    wsb_bytes = lp.lp_lm_head_workspace_bytes(cfg.T, cfg.h, cfg.V, cfg.tile_rows, True)
    wsf = torch.empty(wsf_bytes, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(wsb_bytes, dtype=torch.uint8, device="cuda")
    out = {}

    def step():
        lpv, Hv, lse = lp.lp_lm_head_logprobs_entropy(hid, W, y, m, cfg.temperature, cfg.tile_rows, workspace=wsf)
        out["g"] = lp.lp_lm_head_logprobs_entropy_backward(hid, W, y, m, cfg.temperature, cfg.tile_rows, lse, Hv,
                                                           glp, gH, workspace=wsb)
        out["f"] = (lpv, Hv, lse)

    gemms = ("k_fwd_tile", "k_bwd_dz", "k_out_gemm_dhidden", "k_out_gemm_dweight")
    kernels = list(gemms) + ["k_gather_rows", "k_splitk_reduce", "k_fwd_merge", "k_compact",
                             "k_zero_unscored_rows", "k_transpose_bf16"]
    ms, kt = _timed(lp, torch, step, steps, warmup, kernels)
    power = kt.pop("_power")
    flop_step = 8.0 * Ts * cfg.V * cfg.h
    mfma_ms = sum(kt[k][1] for k in gemms)
    achieved = flop_step * steps / (mfma_ms * 1e-3) / 1e12
    # HBM traffic of the GEMMs per step from the PMC summary (per-launch bytes x launches per step)
    traffic = None
    per = [measured_traffic(k) for k in gemms]
    if all(p is not None for p in per):
        traffic = sum(p * kt[k][0] / steps for p, k in zip(per, gemms))
    res = dict(
        workload=f"fused LM-head forward + recompute backward: T={cfg.T} packed rows ({Ts} scored), h={cfg.h}, "
                 f"V={cfg.V}, bf16, tau {cfg.temperature}, tile {cfg.tile_rows}, dHidden and dW in fp32",
        ms_per_step=ms / steps, tokens_per_s=Ts * steps / (ms * 1e-3),
        frac_of_peak_per_step=flop_step / (ms / steps * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        roofline=dict(bound="mfma", kernel="all MFMA GEMMs (fwd + dZ recompute + dHidden + dW)", achieved=achieved,
                      peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=achieved / BF16_PEAK_TFLOPS, traffic=traffic,
                      traffic_unit="HBM bytes per step of the four GEMM kinds (FETCH_SIZE + WRITE_SIZE, "
                                   "copy-calibrated)",
                      algorithmic_flop_per_step=flop_step,
                      per_gemm_frac={k: (2.0 * Ts * cfg.V * cfg.h) * steps / (kt[k][1] * 1e-3) / 1e12
                                     / BF16_PEAK_TFLOPS for k in gemms},
                      board_power_during_timed_steps=power),
        kernel_ms_per_step={k: v[1] / steps for k, v in kt.items()},
        launches_per_step={k: v[0] / steps for k, v in kt.items()})
    fwd_mem = _memory_audit(torch, lambda: lp.lp_lm_head_logprobs_entropy(hid, W, y, m, cfg.temperature,
                                                                          cfg.tile_rows),
                            wsf_bytes, 3 * 4 * cfg.T, 4 * cfg.T * cfg.V)
    lpv, Hv, lse = out["f"]
    bwd_mem = _memory_audit(torch, lambda: lp.lp_lm_head_logprobs_entropy_backward(
        hid, W, y, m, cfg.temperature, cfg.tile_rows, lse, Hv, glp, gH), wsb_bytes, 4 * (cfg.T + cfg.V) * cfg.h,
        4 * cfg.T * cfg.V)
    res["memory"] = dict(forward=fwd_mem, backward=bwd_mem)
    if cpu_seconds > 0:
        from oracle import lp_oracle as O  # CPU-baseline leg only
        Wl = _LazyWeight(O, A["weight"])
        dH_gpu = out["g"][0]

        def run(rows):
            # the oracle's per-row work of a forward + backward: logits, dZ, the rows' dHidden and their share
            # of dW (formed block by block and dropped: dW sums over every row of the step)
            Hr = O.widen_bf16(A["hidden"][rows])
            _, dZ = O.lm_head_logit_grad(Hr, Wl, A["targets"][rows], None, cfg.temperature,
                                         A["grad_logprob"][rows], A["grad_entropy"][rows])
            dH = np.zeros((len(rows), cfg.h))
            for j0 in range(0, cfg.V, 16384):
                blk = dZ[:, j0:j0 + 16384]
                dH += blk @ Wl[j0:j0 + 16384]
                _ = blk.T @ Hr
            return dH

        rows, t, dH_o = _oracle_timed(np, run, np.nonzero(A["mask"])[0], cpu_seconds, 8)
        got = dH_gpu[torch.as_tensor(rows, device="cuda")].double().cpu().numpy()
        rel_fro = float(np.linalg.norm(got - dH_o) / np.linalg.norm(dH_o))
        rel_max = float(np.abs(got - dH_o).max() / np.abs(dH_o).max())
        res["cpu_baseline"] = _baseline(
            len(rows), t, "scored tokens/s",
            f"{len(rows)} scored rows of the same workload through the fp64 oracle's forward + backward "
            f"(logits, dZ, the rows' dHidden and their dW share; full V={cfg.V}, h={cfg.h})",
            max(rel_fro, rel_max), 1e-2, parity_metric="dHidden rows: max of relative Frobenius and "
                                                       "max|diff| / max|ref|")
    del hid, W, y, m, glp, gH, wsf, wsb, out
    torch.cuda.empty_cache()
    return res


def bench_kl_lm_head(lp, torch, np, synth, steps, warmup, cpu_seconds):
    """KL(teacher || student) rebuilt through both heads: forward timed over
    `steps`, forward + student backward over max(1, steps // 5)."""
    cfg = synth.KLHeads(grads=True).build()
    A = cfg.arrays
    heads = [to_dev_bits(A[k], "bf16") for k in ("student_hidden", "student_weight", "teacher_hidden",
                                                  "teacher_weight")]
    y, dm, g = to_dev(A["targets"]), to_dev(A["diff_mask"]), to_dev(A["grad_kl"])
    wsf_bytes = lp.lp_lm_head_kl_workspace_bytes(cfg.T, cfg.h, cfg.V, cfg.tile_rows, False)
    wsb_bytes = lp.lp_lm_head_kl_workspace_bytes(cfg.T, cfg.h, cfg.V, cfg.tile_rows, True)
    wsf = torch.empty(wsf_bytes, dtype=torch.uint8, device="cuda")
    wsb = torch.empty(wsb_bytes, dtype=torch.uint8, device="cuda")
    out = {}

    def fwd():
        out["f"] = lp.lp_lm_head_kl(*heads, None, y, dm, cfg.tile_rows, workspace=wsf)

    def fwd_bwd():
        fwd()
        out["g"] = lp.lp_lm_head_kl_backward(*heads, None, cfg.tile_rows, out["f"][4], out["f"][5], g,
                                             workspace=wsb)

    ms, kt = _timed(lp, torch, fwd, steps, warmup, ["k_kl_teacher", "k_kl_student", "k_kl_merge"])
    power = kt.pop("_power")
    n_launch, t_ms = kt["k_kl_teacher"]
    s_ms = kt["k_kl_student"][1]
    kms = t_ms + s_ms
    flop_fwd = 2.0 * cfg.T * cfg.V * (cfg.h + cfg.h)
    achieved = flop_fwd * steps / (kms * 1e-3) / 1e12
    chunks = n_launch / steps  # row chunks per forward: one teacher and one student launch each
    chunk_rows = cfg.T / chunks
    # per chunk and pass: one model's weight once, the chunk's hidden rows, the chunk's fp32 teacher logits
    # (written by the teacher pass, read by the student pass)
    pass_bytes = cfg.V * cfg.h * 2 + chunk_rows * cfg.h * 2 + chunk_rows * cfg.V * 4
    bsteps = max(1, steps // 5)
    bkernels = ["k_kl_teacher", "k_kl_student", "k_kl_dz", "k_out_gemm_dhidden", "k_out_gemm_dweight",
                "k_gather_rows", "k_splitk_reduce", "k_transpose_bf16"]
    ms_b, kt_b = _timed(lp, torch, fwd_bwd, bsteps, min(1, warmup), bkernels)
    power_b = kt_b.pop("_power")
    flop_fb = flop_fwd * 2 + 4.0 * cfg.T * cfg.V * cfg.h
    mfma_ms = sum(kt_b[k][1] for k in bkernels[:5])
    achieved_b = flop_fb * bsteps / (mfma_ms * 1e-3) / 1e12
    res = dict(
        workload=f"KL(teacher||student) with logits rebuilt through both heads: T={cfg.T} rows, "
                 f"h_student=h_teacher={cfg.h}, V={cfg.V}, bf16, tile {cfg.tile_rows}, + target lps and prob diff",
        ms_per_step=ms / steps, tokens_per_s=cfg.T * steps / (ms * 1e-3),
        roofline=dict(bound="mfma", kernel="k_kl_teacher + k_kl_student", achieved=achieved,
                      peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=achieved / BF16_PEAK_TFLOPS,
                      traffic=measured_traffic("k_kl_student"),
                      traffic_kernel="k_kl_student",
                      traffic_unit="HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                      traffic_teacher=measured_traffic("k_kl_teacher"),
                      algorithmic_hbm_bytes_per_launch=pass_bytes,
                      launches_per_step=n_launch / steps, algorithmic_flop_per_step=flop_fwd,
                      algorithmic_flop_per_launch=flop_fwd / 2 / chunks,
                      teacher_ms_per_launch=t_ms / n_launch, student_ms_per_launch=s_ms / n_launch,
                      board_power_during_timed_steps=power),
        fwd_bwd=dict(ms_per_step=ms_b / bsteps, tokens_per_s=cfg.T * bsteps / (ms_b * 1e-3),
                     roofline=dict(bound="mfma", kernel="all MFMA GEMMs (2 fwd + 2 recompute + dHidden + dW)",
                                   achieved=achieved_b, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                                   frac=achieved_b / BF16_PEAK_TFLOPS, algorithmic_flop_per_step=flop_fb,
                                   board_power_during_timed_steps=power_b),
                     kernel_ms_per_step={k: v[1] / bsteps for k, v in kt_b.items()}))
    res["memory"] = _memory_audit(torch, lambda: lp.lp_lm_head_kl(*heads, None, y, dm, cfg.tile_rows), wsf_bytes,
                                  6 * 4 * cfg.T, 2 * 4 * cfg.T * cfg.V)
    if cpu_seconds > 0:
        from oracle import lp_oracle as O  # CPU-baseline leg only
        got = [t.cpu().numpy() for t in out["f"]]
        Ws, Wt = _LazyWeight(O, A["student_weight"]), _LazyWeight(O, A["teacher_weight"])

        def run(rows):
            return O.lm_head_kl(O.widen_bf16(A["student_hidden"][rows]), Ws, O.widen_bf16(A["teacher_hidden"][rows]),
                                Wt, None, A["targets"][rows], A["diff_mask"][rows])

        rows, t, want = _oracle_timed(np, run, np.arange(cfg.T), cpu_seconds, 8)
        err = max(np.abs(gv[rows] - w).max() for gv, w in zip(got, want))
        res["cpu_baseline"] = _baseline(len(rows), t, "tokens/s",
                                        f"{len(rows)} rows of the same workload through the fp64 oracle (both "
                                        f"heads' logits, full V={cfg.V}, h={cfg.h}; forward)", err, 2e-3)
    del heads, y, dm, g, wsf, wsb, out
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# second denominators: what this GPU reaches
# ---------------------------------------------------------------------------

def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "entropy_chunked_row_amd", "liblp_probe.so")
    if not os.path.exists(path):
        return None
    probe = ctypes.CDLL(path)
    probe.lp_probe_read.restype = ctypes.c_int
    probe.lp_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.lp_probe_mfma.restype = ctypes.c_int
    probe.lp_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    probe.lp_probe_exp.restype = ctypes.c_int
    probe.lp_probe_exp.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    probe.lp_probe_clock_rates.restype = ctypes.c_int
    probe.lp_probe_clock_rates.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    return probe


def _clocked_probe(torch, probe, fn, iters, per_cu=1):
    """Runs a liblp_probe.so kernel that records clock pairs (per_cu
    workgroups per CU) for SETTLE_SECONDS, then three timed launches; returns
    the best launch time (ms) and the shader clock (MHz) its workgroups ran at
    (ratio of the shader-clock and fixed-frequency counters read inside the
    launch)."""
    import ctypes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = per_cu * cus
    clocks = torch.zeros(4 * blocks, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def run():
        assert fn(blocks, iters, clocks.data_ptr(), sink.data_ptr(), stream) == 0

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_SECONDS:
        run()
        torch.cuda.synchronize()
    best, sclk = None, None
    wall, peak = ctypes.c_int(0), ctypes.c_int(0)
    rates_ok = probe.lp_probe_clock_rates(ctypes.byref(wall), ctypes.byref(peak)) == 0
    for _ in range(3):
        ms = _events_ms(torch, run, 1)
        if best is None or ms < best:
            best = ms
            c = clocks.cpu().numpy().reshape(-1, 4).astype("float64")
            dt, dr = c[:, 1] - c[:, 0], c[:, 3] - c[:, 2]
            if rates_ok and (dr > 0).all():
                sclk = float((dt / dr).mean() * wall.value / 1e3)  # MHz
    del clocks, sink
    return best, sclk, cus, (peak.value / 1e3 if rates_ok else None)


def measure_mfma(torch, probe):
    """Back-to-back v_mfma_f32_32x32x16_bf16 at two waves per SIMD on every CU
    (liblp_probe.so), after SETTLE_SECONDS of the same work: the best of three
    timed launches, and the shader clock the matrix cores ran at."""
    iters = 200000
    ms, sclk, cus, peak = _clocked_probe(torch, probe, probe.lp_probe_mfma, iters)
    flop = cus * 8 * iters * 8 * MFMA_FLOP
    return dict(bf16_mfma_tflops=flop / (ms * 1e-3) / 1e12, mfma_probe_sclk_mhz=sclk, peak_sclk_mhz=peak,
                mfma_probe=f"{cus} workgroups x 8 waves x {iters} x 8 back-to-back v_mfma_f32_32x32x16_bf16 "
                           "(two waves per SIMD), best of 3 after the settle")


def measure_exp(torch, probe):
    """Back-to-back v_exp_f32 (sixteen independent chains per lane, two
    workgroups of 16 waves per CU, so every SIMD holds 8 waves whatever CU the
    dispatcher picks): the transcendental rate the row kernels draw on, one
    exp2 per logit."""
    iters = 20000
    ms, sclk, cus, _ = _clocked_probe(torch, probe, probe.lp_probe_exp, iters, per_cu=2)
    n = 2 * cus * 1024 * iters * 16
    rate = n / (ms * 1e-3)
    return dict(exp2_per_s=rate, exp_probe_sclk_mhz=sclk,
                exp2_per_clk_per_cu=(rate / (sclk * 1e6) / cus) if sclk else None,
                exp_probe=f"{2 * cus} workgroups x 1024 lanes x {iters} x 16 back-to-back v_exp_f32, best of 3")


def measure_achievable(torch):
    """Second denominators beside the datasheet peaks, measured on this GPU:
    the read bandwidth of a streaming read of 4 GiB, the bf16 matrix-core rate
    of back-to-back MFMAs and the v_exp_f32 rate (all from the bench-only
    liblp_probe.so), and, as context, a large library bf16 GEMM (torch.matmul,
    8192^3)."""
    out = dict(hbm_read_gbs=None, bf16_mfma_tflops=None, mfma_probe_sclk_mhz=None, bf16_gemm_tflops=None,
               source="liblp_probe.so: streaming read of 4 GiB (best of 5 grid sizes), back-to-back MFMAs, "
                      "back-to-back v_exp_f32; "
                      "torch.matmul bf16 8192^3 (library GEMM, context only)")
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)

    def gemm():
        torch.matmul(a, b)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_SECONDS:
        gemm()
        torch.cuda.synchronize()
    gemm_ms = min(_events_ms(torch, gemm, 10) / 10 for _ in range(3))
    out["bf16_gemm_tflops"] = 2.0 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12
    del a, b
    probe = _probe_lib()
    if probe is not None:
        out.update(measure_mfma(torch, probe))
        out.update(measure_exp(torch, probe))
        nbytes = 4 << 30
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        best = None
        for blocks in (4096, 8192, 14134, 16384, 32768):
            def read():
                assert probe.lp_probe_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), stream) == 0
            read()
            ms = min(_events_ms(torch, read, 5) / 5 for _ in range(2))
            gbs = nbytes / (ms * 1e-3) / 1e9
            best = gbs if best is None or gbs > best else best
        out["hbm_read_gbs"] = best
        del buf, sink
    torch.cuda.empty_cache()
    return out


def _add_achievable(roof, ach):
    if not roof or roof.get("achieved") is None:
        return
    if roof.get("unit") == "GB/s":
        ref = ach.get("hbm_read_gbs")
        if ach.get("exp2_per_s"):
            # the row kernels evaluate one exp2 per 2-byte logit they read: the share of the
            # transcendental rate the probe measured that the achieved bandwidth draws on
            roof["exp2_share_of_probe_rate"] = roof["achieved"] * 1e9 / 2 / ach["exp2_per_s"]
    else:
        ref = ach.get("bf16_mfma_tflops")
        if ach.get("bf16_gemm_tflops"):
            roof["frac_of_library_gemm"] = roof["achieved"] / ach["bf16_gemm_tflops"]
    if ref:
        roof["frac_of_achievable"] = roof["achieved"] / ref


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--paths", default="all", help="comma list of " + ",".join(ALL_PATHS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the headline path's oracle CPU baseline (0 = skip every CPU baseline)")
    ap.add_argument("--cpu-seconds-path", type=float, default=6.0,
                    help="budget of each other path's oracle CPU baseline")
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="untimed seconds of each path's step before its warm-up steps (steady GPU clocks)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (reference for HBM counters)")
    ap.add_argument("--no-achievable", action="store_true", help="skip the probes (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(rows would shard across GPUs with no exchange in the forward paths)", file=sys.stderr)
        sys.exit(2)
    paths = ALL_PATHS if args.paths == "all" else tuple(p.strip() for p in args.paths.split(","))
    global SETTLE_SECONDS
    SETTLE_SECONDS = max(0.0, args.settle_seconds)

    import numpy as np
    import torch

    import entropy_chunked_row_amd as lp
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lp.load()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst
        torch.cuda.empty_cache()
    head_key = "lm_head_fwd" if "lm_head_fwd" in paths else paths[0]
    cpu_head = args.cpu_seconds
    cpu_path = args.cpu_seconds_path if args.cpu_seconds > 0 else 0.0
    results = {}
    for p in paths:
        log(f"path {p}: building inputs and timing")
        t0 = time.time()
        cs = cpu_head if p == head_key else cpu_path
        if p == "lm_head_fwd":
            results[p] = bench_lm_head_fwd(lp, torch, np, synth, args.steps, args.warmup, cs)
        elif p == "tiny_lm_head":
            results[p] = bench_tiny_lm_head(lp, torch, np, synth, args.steps, args.warmup, cs)
        elif p == "logits_input":
            results[p] = bench_logits_input(lp, torch, np, synth, args.steps, args.warmup, cs)
        elif p == "kl_prob_diff":
            results[p] = bench_kl(lp, torch, np, synth, args.steps, args.warmup, cs)
        elif p == "kl_lm_head":
            results[p] = bench_kl_lm_head(lp, torch, np, synth, args.steps, args.warmup, cs)
        elif p == "lm_head_fwd_bwd":
            results[p] = bench_lm_head_fwd_bwd(lp, torch, np, synth, max(1, args.steps // 5), min(1, args.warmup),
                                               cs)
        else:
            raise SystemExit(f"unknown path {p}")
        log(f"path {p}: done in {time.time() - t0:.1f}s: {results[p]['tokens_per_s']:.4g} tok/s, "
            f"{results[p]['ms_per_step']:.3f} ms/step")

    ach = {} if args.no_achievable else measure_achievable(torch)
    if ach:
        log(f"achievable on this GPU: {ach['hbm_read_gbs'] or 0:.0f} GB/s read, "
            f"{ach['bf16_mfma_tflops'] or 0:.0f} TFLOP/s bf16 MFMA at {ach['mfma_probe_sclk_mhz'] or 0:.0f} MHz, "
            f"library GEMM {ach['bf16_gemm_tflops']:.0f} TFLOP/s")
    for r in results.values():
        _add_achievable(r.get("roofline"), ach)
        _add_achievable(r.get("fwd_bwd", {}).get("roofline"), ach)
    head = results[head_key]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "scored tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_seconds": SETTLE_SECONDS,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "path": head_key},
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "memory": head.get("memory"),
        "achievable": ach,
        "paths": {k: v for k, v in results.items() if k != head_key},
        "parity": {k: {f: v for f, v in r["cpu_baseline"].items() if f.startswith("parity")}
                   for k, r in results.items() if r.get("cpu_baseline")},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
