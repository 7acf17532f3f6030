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


def _layout_bytes(spec, step, k=None):
    """The bytes a step (and, with k, a fold of k live tokens first) must move,
    counted from the synthetic data structures themselves: a slot's packed
    checkpoint page (+ its scale page: fp8 row scales, nvfp4 block scales and
    the slot's second-level scale word), one ring row of each ring tensor
    (page size / L), the step's input arrays and its output rows."""
    L = spec.ring_len
    ckpt = spec.state_bytes()
    if spec.state_dtype == "fp8":
        ckpt += spec.scale_bytes()
    if spec.state_dtype == "nvfp4":
        ckpt += spec.scale_bytes() + 4
    ring_row = spec.x_bytes() // L + spec.B_bytes() // L + spec.dt_bytes() // L
    tokens = step.tokens
    inputs = step.x.nbytes + step.B.nbytes + step.C.nbytes + step.dt.nbytes
    out = tokens * spec.nheads * spec.headdim * 2
    appends = tokens * ring_row
    live = step.pnat if k is None else step.pnat - k
    total = inputs + out + appends + sum(ckpt + int(p) * ring_row for p in live)
    if k is not None:  # the fold: the checkpoint written back and its k ring rows read; its read is shared
        total += sum(ckpt + int(kk) * ring_row for kk in k if kk > 0)
    return total


def test_byte_counts_from_the_data_layouts():
    """bench.py's algorithmic bytes for a plain step, a flush and a fused step
    against a count taken from the synthetic layouts (several state types,
    varlen entries, live rings, folds of 0..pnat tokens)."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    for state in ("f32", "bf16", "f16", "fp8", "nvfp4"):
        spec = synth.CacheSpec(num_slots=40, nheads=32, ngroups=4, state_dtype=state,
                               separate=(state == "nvfp4"))
        step = synth.make_step(spec, 24, 6, 11, 8, varlen=True)
        Tb = np.diff(step.cu_seqlens)
        H, G = spec.nheads, spec.ngroups
        assert bench.step_bytes(spec, H, G, step.pnat, Tb) == _layout_bytes(spec, step), state
        k = np.array([int(p) // 2 for p in step.pnat], np.int32)
        ckpt_rw = sum(1 for kk in k if kk > 0)
        flush_want = _layout_bytes(spec, step, k) - _layout_bytes(spec, step.__class__(
            **{**step.__dict__, "pnat": step.pnat - k}))
        # a flush alone also reads each folded checkpoint (the fused step shares that read)
        per_ckpt = bench.state_bytes(spec, H)
        assert bench.flush_bytes(spec, H, G, k) == flush_want + ckpt_rw * per_ckpt, state
        fused = _layout_bytes(spec, step.__class__(**{**step.__dict__, "pnat": k.copy()}), k)
        assert bench.fused_bytes(spec, H, G, k, Tb) == fused, state
