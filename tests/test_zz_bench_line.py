"""bench.py end to end on the GPU, with the arguments an outside harness passes
(--gpus 1 --steps 20 --warmup 5): exit status 0 and one JSON line whose fields keep
their contract. Named to run last: a failure here hides no parity test under -x."""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def _run_bench(*args, timeout=300):
    print(f"[gpu] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, f"bench.py exited {r.returncode}:\n{r.stderr[-2000:]}"
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, f"expected one JSON line, got {len(lines)}:\n{r.stdout[-2000:]}"
    return json.loads(lines[0])


def test_bench_line_contract():
    d = _run_bench("--gpus", "1", "--steps", "20", "--warmup", "5")
    # the GDN workload, whole windows of 8 steps: 20 -> 24 timed, 5 -> 8 warmup
    assert d["metric"].startswith("decode steps/sec")
    assert d["unit"] == "decode steps/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["scaling"] == "weak" and d["data"] == "synthetic"
    assert (d["steps"], d["warmup"]) == (24, 8)
    assert (d["steps_requested"], d["warmup_requested"]) == (20, 5)
    assert d["vs_baseline"] is None
    cfg = d["config"]
    assert (cfg["rule"], cfg["batch"], cfg["heads"], cfg["d_k"], cfg["d_v"], cfg["window"],
            cfg["rank"]) == ("gdn", 256, 32, 128, 128, 8, 8)
    assert "workload" in cfg
    assert d["value"] > 0 and math.isfinite(d["value"])
    # the timed region is what ms_per_step x steps says it is
    assert d["ms_per_step"] == pytest.approx(1e3 / d["value"], rel=1e-9)
    assert d["ms_per_step"] * d["steps"] / 1e3 < d["bench_wall_s"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["launches"] == 3  # one update + refresh per timed window
    # algorithmic bytes of one launch: 8192 units x (8 d_k d_v + 4 r d_v + W x 520) bytes
    assert rf["bytes_per_launch"] == 8192 * (8 * 128 * 128 + 4 * 8 * 128 + 8 * 520)
    assert rf["achieved"] == pytest.approx(rf["bytes_per_launch"] / (rf["avg_launch_ms"] * 1e-3)
                                           / 1e9, rel=1e-9)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    assert 0.0 < rf["frac"] <= 1.0
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "decode steps/s"
    assert cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
    # the approximation error of the sketch read against the exact read is reported
    err = d["approx_error"]["projection"]
    assert 0.0 < err["frobenius"] < 2.0 and err["vectors"] > 0

