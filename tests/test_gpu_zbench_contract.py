"""bench.py's output contract: one JSON line with the throughput of the decode
step, the dominant kernel's roofline figures and the CPU oracle's rate.

The CPU test checks the one-GPU refusal, which happens before anything
touches a GPU.  The GPU test runs a short bench in a child process (the
default kpa_32k workload: 32 sequences x 32768 cached tokens, one query each)
and checks the line's fields against each other.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    res = subprocess.run([sys.executable, BENCH, *argv], capture_output=True, text=True, timeout=60,
                         env={**os.environ, **env}, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_json_line_is_consistent(tmp_path):
    out = tmp_path / "bench.json"
    cmd = [sys.executable, "-u", BENCH, "--steps", "4", "--warmup", "2", "--cpu-seconds", "1",
           "--json-out", str(out)]
    print("running", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.strip().splitlines() if ln.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    d = json.loads(lines[0])

    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["dtype"] == "bf16"
    assert d["unit"] == "cached tokens/s"
    cfg = d["config"]
    assert cfg["workload"] == "kpa_32k" and cfg["batch"] == 32 and cfg["ctx"] == 32768 and cfg["n_q"] == 1
    assert cfg["path"] == "mfma_bf16"
    # whole-step throughput: every cached token of every sequence per step
    assert d["ms_per_step"] > 0
    assert d["value"] == pytest.approx(32 * 32768 / (d["ms_per_step"] * 1e-3), rel=1e-3)

    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    # per cached token (R_K + R_V)(p1 q1 + p2 q2) bf16 elements = 4 * (32 + 64) * 2
    # = 768 B; per sequence the float32 query, output and lse of 16 heads of
    # 128 features, and the fused append's new token (768 B read, 768 B
    # written, its position and slot)
    assert r["alg_bytes_per_launch"] == (32 * 32768 * 768 + 32 * 16 * (2 * 128 + 1) * 4
                                         + 32 * (2 * 768 + 4 + 4))
    assert r["achieved"] == pytest.approx(r["alg_bytes_per_launch"] / (r["launch_us"] * 1e-6) / 1e9, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    assert 0.0 < r["frac"] < 1.0
    # the kernel runs inside the step
    assert r["launch_us"] * 1e-3 < d["ms_per_step"]
    if r["traffic"] is not None:
        assert r["traffic"] >= r["alg_bytes_per_launch"] * 0.9

    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == d["unit"]
    assert c["value"] > 0 and c["cores"] >= 1 and isinstance(c["sample"], str)

    assert json.loads(out.read_text().strip().splitlines()[-1]) == d
