"""bench.py's output contract, on the GPU: a short run of the default command
prints one JSON line with every field the line promises (the metric, the
timing protocol, the roofline of the dominant kernel with its HBM traffic
field, the launch floor, the plain HBM streams, the fp8 loop as the extra
record and the CPU oracle beside it), with values that hang together."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bench_line_contract():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1", "--trials", "2",
           "--settle", "0.2", "--cpu-seconds", "0.5"]
    print("bench:", " ".join(cmd[1:]), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, p.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "timing", "roofline", "launch_floor_us", "hbm_stream",
              "extra", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["unit"] == "tokens/s" and d["value"] > 0 and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("large")
    assert d["timing"]["trials"] == 2
    tokens_per_s = d["config"]["tokens_per_step"] / (d["ms_per_step"] * 1e-3)
    assert abs(tokens_per_s - d["value"]) <= 1e-6 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000
    assert 0 < r["achieved"] < r["peak"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert r["traffic"] is None or r["traffic"] > 0
    assert 0 < d["launch_floor_us"] < 100
    for k in ("copy_GBps", "rmw_GBps", "write_GBps", "read_GBps"):
        assert 0 < d["hbm_stream"][k] < 8000, k
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    assert "fp8_fused_flush" in d["extra"]
