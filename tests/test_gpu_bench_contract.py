"""bench.py's output line on the GPU: one JSON object with every field the
benchmark contract names, numbers that agree with each other, and the
oracle's CPU rate beside the GPU's.  A few short steps of the default
workload (the 70B-shaped GQA layer, with the other decode workloads under
"also") and of one several-token workload."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

TOP_FIELDS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"}
ROOFLINE_FIELDS = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


def _bench(*args):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def test_default_decode_line():
    res = _bench("--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5")
    assert TOP_FIELDS <= set(res)
    assert res["n_gpus"] == 1 and res["steps"] == 3 and res["warmup"] == 1
    assert res["higher_is_better"] is True and res["unit"] == "GB/s" and res["dtype"] == "bf16"
    assert res["vs_baseline"] is None
    assert "workload" in res["config"] and "model" not in res["config"]
    # value = distinct K/V bytes of the step / step time
    kv = res["config"]["kv_bytes"]
    assert res["value"] == pytest.approx(kv / (res["ms_per_step"] * 1e-3) / 1e9, rel=2e-3)
    roof = res["roofline"]
    assert ROOFLINE_FIELDS <= set(roof)
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    # the kernel runs inside the step
    assert 0 < roof["avg_launch_us"] < res["ms_per_step"] * 1e3
    assert roof["achieved"] == pytest.approx(roof["algorithmic_bytes_per_launch"] / (roof["avg_launch_us"] * 1e-6) / 1e9,
                                             rel=1e-3)
    cpu = res["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert cpu["sample"]
    # the copy kernel's bandwidth on the same box, and the clocks seen under load
    assert res["calibration"]["copy_read_plus_write_GBs"] > 0
    assert "clocks" in res["env"]
    # the other decode workloads of the same process
    also = res["also"]
    assert [(a["config_id"], bool(a["shared_prefix"])) for a in also] == [(2, False), (4, False), (4, True),
                                                                          (5, False)]
    for a in also:
        assert a["value"] == pytest.approx(a["kv_bytes"] / (a["us_per_step"] * 1e-6) / 1e9, rel=2e-3)
        assert 0 < a["roofline"]["frac"] < 1 and 0 < a["roofline"]["avg_launch_us"] < a["us_per_step"]


def test_several_token_line():
    res = _bench("--extend", "verify", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    assert TOP_FIELDS <= set(res)
    roof = res["roofline"]
    assert ROOFLINE_FIELDS <= set(roof)
    assert roof["bound"] in ("hbm", "mfma")
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert 0 < roof["avg_launch_us"] < res["ms_per_step"] * 1e3
