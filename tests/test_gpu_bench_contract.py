"""bench.py's output line on the GPU: one JSON object with the fields its readers rely on, and
figures that agree with each other (the step rate with the step's FLOP count, the roofline fraction
with the attention kernel's bytes and time, the CPU baseline's description).

bench.py runs as a child process with a short timed region (3 steps, one input set, a 1-second CPU
sample), so this checks the contract, not the performance.
"""
import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the decode step at B=32, n_h=128, 4096 tokens: per cached token and head a 576-wide score and a
# 512-wide weighted sum, per sequence and head the W_UK absorption and the W_UV up-projection
STEP_FLOP = 32 * (4096 * 128 * 2 * (576 + 512) + 128 * 2 * (128 * 512 * 2))
CACHE_BYTES = 32 * 4096 * 1152


def test_bench_line_contract():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", "--sets", "1",
           "--cpu-seconds", "1"]
    say(f"[bench contract] {' '.join(cmd[1:])}")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])

    assert d["metric"] and d["unit"] == "TFLOP/s" and d["value"] > 0
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 1)
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert "workload" in d["config"] and d["config"]["global_batch"] == 32 and d["config"]["seq_len"] == 4096
    # the rate is the step's algorithmic FLOP over the step time (both rounded in the line)
    rate = STEP_FLOP / (d["ms_per_step"] * 1e-3) / 1e12
    assert abs(rate - d["value"]) <= 1e-3 * d["value"] + 0.01, (rate, d["value"])

    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["algorithmic_bytes_per_launch"] == CACHE_BYTES
    achieved = CACHE_BYTES / (d["kernels_ms"]["decode_attention"] * 1e-3) / 1e9
    assert abs(achieved - rf["achieved"]) <= 2e-3 * rf["achieved"], (achieved, rf["achieved"])
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) <= 1e-4
    assert 0 < rf["frac"] < 1
    # measured HBM bytes per launch, when present: at least the cache, well under twice it
    assert rf["traffic"] is None or CACHE_BYTES <= rf["traffic"] < 2 * CACHE_BYTES

    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["unit"] == "TFLOP/s"
    assert isinstance(cb["cores"], int) and cb["cores"] >= 1 and cb["sample"]
    say(f"  value {d['value']} TFLOP/s, {d['ms_per_step'] * 1e3:.1f} us per step, attention {rf['frac']:.3f} of HBM")
