"""Host-side parts of bench.py (no GPU): the one-GPU guard, the algorithmic byte counts the
roofline and stage rates divide by, and the traffic record's bookkeeping."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_algorithmic_bytes_at_the_video_shape():
    """Pass 2: bf16 Q/K read + write, fp32 cos and sin rows, the two sums per token and the two
    gammas; producer: hidden + residual read, residual sum written, ROW_MX rows (H codes + fp32
    scale) or MX rows (H codes + H / 32 exponents) written, gamma read."""
    p = synth.CONFIGS[5].calls[0]
    T, H, Iq, Ik, d = p.T, p.H, p.Iq, p.Ik, p.head_dim
    assert (T, H, Iq, Ik, d) == (75600, 5120, 5120, 5120, 128)
    b = bench.algorithmic_bytes(p, producer=True)
    assert b["norm_rope"] == 4 * T * (Iq + Ik) + 8 * T * d + 8 * T + 2 * (Iq + Ik)
    assert b["norm_rope"] == pytest.approx(3.175e9, rel=2e-4)      # 3.175 GB per step
    assert b["producer"] == 6 * T * H + T * (H + 4) + 2 * H
    assert b["producer"] == pytest.approx(2.710e9, rel=2e-4)       # 2.710 GB per step
    bm = bench.algorithmic_bytes(p, producer=True, mx=True)
    assert bm["producer"] == 6 * T * H + T * (H + H // 32) + 2 * H
    assert bench.algorithmic_bytes(p, producer=False)["producer"] == 0


def test_traffic_record_is_tied_to_the_projection_sources():
    """The committed record names the sources it was measured on; a record with another digest
    is never reported."""
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert set(rec["per_kernel"]) >= {"project_kernel", "ssq_reduce_kernel"}
    assert rec["hbm_bytes_per_call"] == pytest.approx(
        sum(v["read_bytes"] + v["write_bytes"] for v in rec["per_kernel"].values()))
    digest = bench.source_digest(bench.PROJECT_SRC)
    assert len(digest) == 16
    if rec["kernel_src_sha256_16"] == digest:
        assert bench.measured_traffic(bench.STAGED_KERNELS) == pytest.approx(
            rec["hbm_bytes_per_call"])


def test_config_block_entry_divides_by_the_published_peaks():
    """One workload's entry of the per-config block: projection TFLOP/s against 5.0 PFLOP/s,
    norm GB/s against 8 TB/s, nothing recomputed from other fields."""
    p = synth.CONFIGS[2].calls[0]
    r = {"p": p, "ms_per_step": 0.33, "stage_ms": {"projection": 0.28, "norm_rope": 0.04},
         "projection_tflops": 2300.0, "norm_rope_gbs": 4400.0}
    c = bench._compact(r)
    assert (c["T"], c["H"], c["I"]) == (4096, 5120, 15360)
    assert c["projection_frac_of_peak"] == pytest.approx(2300.0 / 5000.0)
    assert c["norm_rope_hbm_frac"] == pytest.approx(4400.0 / 8000.0)
    assert c["projection_ms"] == 0.28 and c["norm_rope_ms"] == 0.04


def test_power_summary_assigns_samples_to_phases(tmp_path, capsys):
    """--summarize-power: samples inside a phase (after its first second) are averaged; samples
    outside every phase and a malformed sample are ignored."""
    import json
    import bench

    def sample(t, watts, clocks):
        g = {"gpu": 0, "power": {"socket_power": {"value": watts, "unit": "W"}},
             "clock": {f"gfx_{i}": {"clk": {"value": c, "unit": "MHz"}} for i, c in enumerate(clocks)}}
        g["clock"]["mem_0"] = {"clk": {"value": 1900, "unit": "MHz"}}
        return f"T {t:.6f}\n" + json.dumps({"gpu_data": [g]}, indent=1) + "\n"

    phases = tmp_path / "phases.log"
    phases.write_text("\n".join(json.dumps(d) for d in [
        {"phase": "a", "start": 100.0}, {"phase": "a", "end": 104.0, "calls": 10, "ms_per_call": 4.0},
        {"phase": "b", "start": 104.0}, {"phase": "b", "end": 108.0, "calls": 5, "ms_per_call": 2.0},
    ]) + "\n[bench] noise\n")
    samples = tmp_path / "samples.txt"
    samples.write_text(sample(100.5, 999, [100, 100])            # a's first second: left out
                       + sample(101.5, 1400, [1700, 1720])
                       + sample(103.0, 1380, [1740, 1760])
                       + "T 103.500000\nnot json\n"
                       + sample(106.0, 700, [2400, 2380])
                       + sample(120.0, 5, [1, 1]))               # after every phase
    out = bench.summarize_power(str(phases), str(samples))
    by = {o["phase"]: o for o in out}
    assert by["a"]["samples"] == 2 and by["a"]["power_w"] == 1390.0
    assert by["a"]["gfx_clock_mhz"] == 1730.0 and by["a"]["ms_per_call"] == 4.0
    assert by["b"]["samples"] == 1 and by["b"]["power_w"] == 700.0 and by["b"]["gfx_clock_mhz"] == 2390.0
