"""The benchmark's result line: one JSON object, short enough to survive a capture that keeps
only the tail of the output, carrying both gated figures (the decode GEMV's HBM fraction with its
traffic, the prefill GEMM's MFMA fraction)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_result_line_is_short_and_complete():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[gpu-case] bench.py short run", flush=True)
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "20", "--warmup", "5", "--no-rows",
           "--no-cpu-baseline", "--prefill-steps", "3", "--sustain", "0.5"]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.strip().splitlines() if l.strip()]
    assert len(lines) == 1, lines
    line = lines[0]
    d = json.loads(line)
    # the default run adds the row count and the oracle's rate (about 150 bytes)
    assert len(line) + 200 < 1500, len(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "prefill_gemm"):
        assert key in d, key
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and 0 < rf["frac"] < 1 and rf["traffic"] is not None
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    pg = d["prefill_gemm"]
    assert 0 < pg["frac"] < 1 and pg["traffic"] is not None
