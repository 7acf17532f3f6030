"""bench.py's command-line contract that holds without a GPU: more than one
GPU is refused with a message (the step has no cross-GPU exchange), and the
algorithmic byte counts follow the per-entry formulas."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_step_bytes_formula():
    """One fp16 entry, H=128, G=8, p live and T new tokens, bf16 output:
    state + live ring (x, B, dt') + new tokens (x, B, C, dt) + output + appends."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    spec = synth.CacheSpec(num_slots=2, nheads=128, ngroups=8, state_dtype="f16")
    H, G, p, T = 128, 8, 3, 8
    want = (H * 64 * 128 * 2 + p * (H * 64 * 2 + G * 128 * 2 + H * 4) + T * (H * 64 * 2 + 2 * G * 128 * 2 + H * 4)
            + T * H * 64 * 2 + T * (H * 64 * 2 + G * 128 * 2 + H * 4))
    got = bench.step_bytes(spec, H, G, np.array([p]), np.array([T]))
    assert got == want
