"""The benchmark's one JSON line at a short run: the keys and types the line
promises, the roofline fraction and scores/s recomputed from the line's own
figures, and the CPU baseline object. The benchmark runs as a child process, as
it does for any caller."""
import json
import math
import os
import subprocess
import sys

import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bench_line_contract():
    say("bench: decode, 20 steps, 5 warmup, 1 s CPU baseline")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20", "--warmup", "5",
                        "--cpu-seconds", "1"], cwd=ROOT, capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(d[key], typ), (key, d.get(key))
    assert "vs_baseline" in d
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5 and d["higher_is_better"] is True
    c = d["config"]
    assert c["workload"] == "decode" and (c["P"], c["B"], c["S"], c["D"]) == (1, 32, 32768, 128)
    # scores per second of the whole step
    assert math.isclose(d["value"], c["P"] * c["B"] * c["S"] / (d["ms_per_step"] * 1e-3), rel_tol=1e-6)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert math.isclose(rf["frac"], rf["achieved"] / rf["peak"], rel_tol=1e-9)
    # achieved = algorithmic bytes of one launch over its event-timed duration
    assert math.isclose(rf["achieved"], rf["bytes_per_launch"] / (rf["avg_launch_us"] * 1e-6) / 1e9, rel_tol=1e-6)
    assert 0.0 < rf["frac"] < 1.0
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == d["unit"]
    say(f"bench: {d['value']:.3g} {d['unit']}, frac {rf['frac']:.3f}, cpu {cb['value']:.3g}")
