"""The benchmark's output contract: one JSON line with the metric, the
whole-job value, the step accounting, the roofline of the dominant kernel and
the CPU baseline; a request for more than one GPU is refused with a message
(checked in a child process, before anything touches a GPU).  The GPU case
runs bench.main() in this process on the tiny workload (a few milliseconds of
GPU work; the oracle sample is a handful of rows)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = r.stdout.strip().splitlines()[-1]
    msg = json.loads(line)["error"]
    assert "one GPU" in msg


@pytest.mark.gpu
def test_json_line_fields(monkeypatch, capsys):
    # in this process (no child process next to one that holds the GPU)
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", [BENCH, "--workload", "1", "--steps", "3", "--warmup", "1", "--cpu-rows", "4"])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1, "bench prints exactly one JSON line"
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 1
    assert out["unit"] == "tokens/s" and out["higher_is_better"] is True
    assert out["value"] > 0 and out["ms_per_step"] > 0
    # value is all positions per second over the timed steps
    assert out["value"] == pytest.approx(out["config"]["N"] / (out["ms_per_step"] * 1e-3), rel=1e-6)
    assert out["dtype"] == "f32" and "workload" in out["config"]
    rf = out["roofline"]
    assert rf["bound"] in ("mfma", "hbm", "alu") and rf["unit"] in ("TFLOP/s", "GB/s")
    assert rf["peak"] > 0 and 0 < rf["frac"] < 1
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    cb = out["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
