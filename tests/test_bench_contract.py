"""bench.py's one-line JSON report: the fields and their consistency (the
roofline fraction is achieved / peak, the CPU baseline is the oracle's, N = 1
only).  The GPU case runs a short benchmark in a child process."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, timeout):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    # answered before any GPU work: one JSON line that says why, nonzero exit
    p = _run(["--gpus", "2"], 120)
    assert p.returncode != 0
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.gpu
def test_report_fields():
    p = _run(["--steps", "2", "--warmup", "1", "--cpu-sample", "48"], 600)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.strip().splitlines() if l.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert k in r, k
    assert r["n_gpus"] == 1 and r["steps"] == 2 and r["warmup"] == 1
    assert r["higher_is_better"] is True and r["vs_baseline"] is None
    assert r["value"] > 0 and r["ms_per_step"] > 0
    # value is entries per second of the timed steps
    assert abs(r["value"] * r["ms_per_step"] / 1e3 / (r["config"]["m"] * r["config"]["n"]) - 1) < 1e-6
    assert "workload" in r["config"]
    rf = r["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 157.3
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert 0 < rf["frac"] < 1
    # the whole band phase: critical and deferred useful flops over both replays
    gp = r["gemm_phase"]
    assert gp["useful_flops"] == r["schedule"]["useful_band_flops"]
    ms = gp["critical_replay_ms"] + gp["deferred_replay_ms"]
    assert abs(gp["tflops"] - gp["useful_flops"] / (ms / 1e3) / 1e12) < 1e-6 * gp["tflops"]
    assert 0 < gp["frac"] < 1
    # the leaf's algorithmic bytes: W in, E, codes, V out, and the lower
    # triangles of the two diagonal factor blocks of each 64 x 64 tile
    assert r["leaf"]["alg_bytes"] == r["config"]["m"] * r["config"]["n"] * (13 + 8 * 2080 / 4096)
    # hessian and factor timed apart from the solve, for both sides
    assert r["hessian_ms"] > 0 and r["factor_ms"] > 0
    assert set(r["prep"]) == {"hessian_A", "factor_A", "hessian_B", "factor_B"}
    cb = r["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cb, k
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert "48x48" in cb["sample"]


@pytest.mark.gpu
def test_report_single_tile_workload():
    # 64 x 64 is one tile diagonal: no band launch, so the band figures are null
    # (and counters from the 4096 x 4096 profile are not attached to it)
    p = _run(["--workload", "c1", "--steps", "2", "--warmup", "1", "--cpu-sample", "16"], 300)
    assert p.returncode == 0, p.stderr[-2000:]
    r = json.loads([l for l in p.stdout.strip().splitlines() if l.startswith("{")][-1])
    assert r["value"] > 0 and r["config"]["m"] == 64
    assert r["roofline"]["achieved"] is None and r["roofline"]["frac"] is None
    assert r["roofline"]["traffic"] is None
    assert r["gemm_phase"]["tflops"] is None and r["gemm_phase"]["frac"] is None
    assert r["leaf"]["launches"] == 1
