"""The benchmark's output contract: one JSON line carrying the metric, the whole-job value, the
timing fields, the dominant kernel's roofline object and the oracle's CPU baseline; more than
one GPU is refused with a message and exit status 2 before anything touches a device."""

import io
import json
import os
import subprocess
import sys
from contextlib import redirect_stdout

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")

TOP_KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
            "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
            "roofline", "cpu_baseline")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _run_main(argv):
    """bench.main() in this process (no child process on a GPU-initialised parent)."""
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    sys.argv = [BENCH] + argv
    buf = io.StringIO()
    try:
        with redirect_stdout(buf):
            bench.main()
    finally:
        sys.argv = old
    lines = [ln for ln in buf.getvalue().splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


@pytest.mark.gpu
@pytest.mark.parametrize("workload", ["d24_short", "d24_decode", "d24_fwd_fp8"])
def test_bench_prints_one_json_line_with_the_contract_fields(workload):
    from gpu_helpers import announce
    announce("bench contract", workload)
    res = _run_main(["--workload", workload, "--steps", "2", "--warmup", "1",
                     "--cpu-seconds", "0.5"])
    for key in TOP_KEYS:
        assert key in res, key
    assert res["n_gpus"] == 1 and res["steps"] == 2 and res["warmup"] == 1
    assert res["value"] > 0 and res["ms_per_step"] > 0
    assert res["higher_is_better"] is True
    assert res["config"]["workload"]
    rl = res["roofline"]
    assert rl["bound"] in ("hbm", "mfma", "alu")
    assert rl["unit"] == ("GB/s" if rl["bound"] == "hbm" else "TFLOP/s")
    assert 0 < rl["frac"] < 1
    assert rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], rel=1e-2, abs=1e-4)
    cb = res["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["sample"]
