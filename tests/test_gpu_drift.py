"""Multi-step drift, reported and not gated.

The fused flush-in-step loop runs for many steps on the GPU from one initial
state. Every step folds the previous step's accepted tokens and reads out T
new ones. Beside it, the oracle runs the same loop in fp64 state mode: its
checkpoint keeps every fold exactly, with no encoding. The error of each
step's outputs against that reference therefore shows how the checkpoint's
encoding compounds over the folds.

Per-call parity elsewhere compares each call with the oracle on the GPU's
own input bytes, so it does not see this growth. The vLLM PR "Add separate
CuTeDSL ReplaySSM checkpoints" (Overview, Claims) keeps an FP16 recurrence
checkpoint with stochastic rounding beside a low-precision read checkpoint,
so that folds do not compound in the read checkpoint's precision. This run
reports the growth for each checkpoint form. It asserts only sanity: finite
outputs, a clean status, and no step's error above ten times the first
step's (plus 0.05).
"""
import numpy as np
import pytest
import torch

import synth
from synth import device as sd

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_harness as gh
    import speculative_replay_state_amd as ssu
from oracle import ssu_oracle as O


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


MODES = {
    "bf16": dict(state="bf16"),
    "fp16": dict(state="f16"),
    "fp8": dict(state="fp8"),
    "fp8_fp16sr": dict(state="fp8", sep=True),
    "nvfp4_fp16sr": dict(state="nvfp4", sep=True),
}
STEPS, BATCH, H, G, T = 32, 16, 16, 2, 4


@pytest.mark.parametrize("mode", list(MODES))
def test_multi_step_drift(mode):
    cfg = MODES[mode]
    spec = synth.CacheSpec(num_slots=BATCH + 1, nheads=H, ngroups=G, state_dtype=cfg["state"],
                           separate=cfg.get("sep", False))
    spec64 = synth.CacheSpec(num_slots=BATCH + 1, nheads=H, ngroups=G, state_dtype="f64")
    rng = np.random.default_rng(77)
    states = (rng.standard_normal((BATCH, H, 64, 128)) * 0.1).astype(np.float32)
    slots = np.arange(1, BATCH + 1, dtype=np.int32)

    t = sd.upload_cache(synth.make_cache(spec, 78), gh.DEV)
    dc = gh.device_cache(spec, t)
    ssu.init_state(dc, torch.from_numpy(states).to(gh.DEV), torch.from_numpy(slots).to(gh.DEV), sr_seed=1)
    ref = synth.make_cache(spec64, 78)
    O.init_state(ref, states, slots)

    first = synth.make_step(spec, BATCH, T, 1000, 0, slots=slots, pnat_fixed=0)
    k = np.zeros(BATCH, np.int32)  # the previous step's accepted tokens, live in the ring
    max_err, rms_err = [], []
    for i in range(STEPS):
        step = synth.make_step(spec, BATCH, T, 1000 + i, 0, slots=slots, pnat_fixed=0)
        step.A[:], step.D[:], step.dt_bias[:] = first.A, first.D, first.dt_bias  # the model's per-head constants
        step.pnat[:] = k
        st = sd.upload_step(step, gh.DEV)
        out = gh.out_tensor(step, spec, "bf16")
        kt = torch.from_numpy(k.copy()).to(gh.DEV)
        desc = ssu.make_step_desc(BATCH, T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"], st["B"],
                                  st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, "bf16", None, "auto",
                                  num_fold=kt, sr_seed=5000 + i)
        ssu.replay_step(dc, desc)
        torch.cuda.synchronize()
        assert int(dc.status.item()) == 0
        r, status = O.replay_step(ref, step, num_fold=k.copy())
        assert status == 0
        got = gh.to_f64(out)
        assert np.all(np.isfinite(got))
        e = np.abs(got - r) / (1.0 + np.abs(r))
        max_err.append(float(e.max()))
        rms_err.append(float(np.sqrt(np.mean(e * e))))
        k = rng.integers(1, T + 1, BATCH).astype(np.int32)

    marks = [0, 3, 7, 15, 31]
    print("drift %-14s max rel err at steps %s: %s; rms: %s" % (
        mode, [m + 1 for m in marks], " ".join("%.2e" % max_err[m] for m in marks),
        " ".join("%.2e" % rms_err[m] for m in marks)), flush=True)
    # sanity only (no blow-up); the growth itself is what this run reports
    assert max(max_err) <= 10.0 * max_err[0] + 0.05
