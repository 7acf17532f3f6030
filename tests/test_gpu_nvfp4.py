"""GPU parity of the NVFP4 read checkpoint (separate checkpoints only).

vLLM PR "Add separate CuTeDSL ReplaySSM checkpoints" (Overview, Claims):
the FP16 recurrence checkpoint is folded in FP32 and written back with
stochastic rounding, the NVFP4 read checkpoint is written with nearest
encoding and read by every step.  Checked through the C ABI against the
oracle: init, flush, the fused step, plain steps (monolith and split, bit for
bit with each other), and the fused step against the GPU's own flush then
step bit for bit.

How an NVFP4 checkpoint written by a fold is checked: the GPU's fp32 fold is
within FOLD_REL * S of the exact one (S the fold of absolute values), and the
GPU encodes its own fp32 values to the nearest point of its own grid, so
every decoded value lies within one element step (e4m3 block scale * g: the
largest half-gap of e2m1, between 4 and 6, also covers saturation at 6) of
the exact fold, plus FOLD_REL * S; the head scale g = max / 2688 moves with
the head maximum.  Most codes and block scales equal the oracle's.
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


def _spec(ring_len=16, num_slots=40, nheads=32, ngroups=4):
    return synth.CacheSpec(num_slots=num_slots, nheads=nheads, ngroups=ngroups, state_dtype="nvfp4",
                           separate=True, ring_len=ring_len)


def _fold_counts(step, seed):
    rng = np.random.default_rng(seed)
    k = np.array([rng.integers(0, int(p) + 1) for p in step.pnat], np.int32)
    k[int(np.argmax(step.pnat))] = int(np.max(step.pnat))
    return k


def test_nvfp4_requires_the_recurrence_checkpoint():
    spec = _spec(num_slots=4, nheads=8, ngroups=1)
    cache = synth.make_cache(spec, 3)
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    dc.recur = None
    ids = torch.zeros(1, dtype=torch.int32, device=gh.DEV)
    with pytest.raises(ssu.SsuError) as e:
        ssu.flush(dc, ids, ids, torch.zeros(8, device=gh.DEV))
    assert e.value.code == ssu.SSU_ERR_UNSUPPORTED


def test_nvfp4_init():
    spec = synth.CacheSpec(num_slots=12, nheads=16, ngroups=2, state_dtype="nvfp4", separate=True, slot_pad=64)
    cache = synth.make_cache(spec, 43)
    rng = np.random.default_rng(8)
    n = 6
    states = (rng.standard_normal((n, 16, 64, 128)) * rng.uniform(0.05, 2.0, (n, 16, 64, 1))).astype(np.float32)
    states[1, 3] = 0.0              # a zero head
    states[2, 0, 5, :16] = 1e-9     # a block far below its head's maximum
    ids = np.array([3, 0, 7, 12, 11, 1], np.int32)
    seed = 0x5EED
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    ssu.init_state(dc, torch.from_numpy(states).to(gh.DEV), torch.from_numpy(ids).to(gh.DEV), sr_seed=seed)
    torch.cuda.synchronize()
    ref = cache.copy()
    O.init_state(ref, states, ids, seed=seed)
    gpu = sd.download_cache(spec, t)
    assert np.array_equal(gpu.recur, ref.recur)
    assert np.array_equal(gpu.gscale, ref.gscale)  # same IEEE division of the same maximum
    assert np.array_equal(gpu.scale, ref.scale)    # same fp32 quotients, nearest e4m3
    # codes: the GPU multiplies by fp32(1 / es) where the oracle divides
    for sl in (3, 7, 11, 1):
        g, r = O.decode_state(gpu, sl), O.decode_state(ref, sl)
        assert np.mean(g == r) >= 0.9999
    for f in ("x_cache", "B_cache", "dt_cache", "ring_start"):
        assert np.array_equal(getattr(gpu, f), getattr(ref, f)), f


@pytest.mark.parametrize("ring_len", [16, 32])
def test_nvfp4_flush_parity(ring_len):
    spec = _spec(ring_len, num_slots=24, nheads=16, ngroups=2)
    cache = synth.make_cache(spec, 51 + ring_len)
    step = synth.make_step(spec, 14, 4, 52, 8)
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, "bf16")
    gh.run_step(dc, st, step, out, "bf16", "monolith")
    ref = cache.copy()
    O.replay_step(ref, step)
    rng = np.random.default_rng(9)
    k = np.array([rng.integers(0, int(p) + 5) for p in step.pnat], np.int32)
    k[0], k[1] = 0, min(int(step.pnat[1]) + 4, spec.ring_len)
    seed = 0xABCDEF
    print("nvfp4 flush", ring_len, "k", k[:8], flush=True)
    ssu.flush(dc, st["slot_idx"], torch.from_numpy(k).to(gh.DEV), st["A"], sr_seed=seed)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    before = ref.copy()
    assert O.flush(ref, step.slot_idx, k, step.A, seed) == 0
    gpu = sd.download_cache(spec, t)
    assert np.array_equal(gpu.ring_start, ref.ring_start)
    touched = sorted({int(s) for s, kk in zip(step.slot_idx, k) if kk > 0})
    gh.check_nvfp4(spec, gpu, ref, before, touched, (step.slot_idx, k, step.A))
    gh.check_recur(spec, gpu, before, step.slot_idx, k, step.A, seed)


def _run_fused(spec, cache, step, k, seed, with_z=False):
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, "bf16")
    desc = ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                              st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, "bf16",
                              None, "auto", num_fold=torch.from_numpy(k).to(gh.DEV),
                              z=st.get("z") if with_z else None, sr_seed=seed)
    ssu.replay_step(dc, desc)
    torch.cuda.synchronize()
    return out, sd.download_cache(spec, t), int(dc.status.item())


@pytest.mark.parametrize("ring_len,with_z", [(16, False), (16, True), (32, False)])
def test_nvfp4_fused_step_parity(ring_len, with_z):
    spec = _spec(ring_len, num_slots=24, nheads=16, ngroups=2)
    cache = synth.make_cache(spec, 61 + ring_len)
    T = 8 if ring_len > 16 else 4
    step = synth.make_step(spec, 13, T, 62, ring_len - T, with_z=with_z)
    k = _fold_counts(step, 63)
    seed = 0x1357
    print("nvfp4 fused", ring_len, with_z, "k", k[:8], flush=True)
    out, gpu, status = _run_fused(spec, cache, step, k, seed, with_z)
    assert status == 0
    ref_cache = cache.copy()
    ref, st = O.replay_step(ref_cache, step, num_fold=k, seed=seed)
    assert st == 0
    gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, "bf16")
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    assert np.array_equal(gpu.x_cache, ref_cache.x_cache)
    assert np.array_equal(gpu.B_cache, ref_cache.B_cache)
    touched = sorted({int(s) for s, kk in zip(step.slot_idx, k) if kk > 0 and 0 < s < spec.num_slots})
    gh.check_nvfp4(spec, gpu, ref_cache, cache, touched, (step.slot_idx, k, step.A))
    gh.check_recur(spec, gpu, cache, step.slot_idx, k, step.A, seed)


def test_nvfp4_fused_equals_gpu_flush_then_step():
    spec = _spec(16, num_slots=24, nheads=16, ngroups=2)
    cache = synth.make_cache(spec, 71)
    step = synth.make_step(spec, 15, 4, 72, 12)
    k = _fold_counts(step, 73)
    seed = 77
    out_f, gpu_f, st_f = _run_fused(spec, cache, step, k, seed)
    assert st_f == 0
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    st = sd.upload_step(step, gh.DEV)
    ssu.flush(dc, st["slot_idx"], torch.from_numpy(k).to(gh.DEV), st["A"], sr_seed=seed)
    step2 = synth.StepInputs(**{**step.__dict__, "pnat": (step.pnat - k).astype(np.int32)})
    st2 = sd.upload_step(step2, gh.DEV)
    out_s = gh.out_tensor(step, spec, "bf16")
    gh.run_step(dc, st2, step2, out_s, "bf16", "monolith")
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    gpu_s = sd.download_cache(spec, t)
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    for f in sd.CACHE_FIELDS + ("recur", "gscale", "ring_start"):
        assert np.array_equal(getattr(gpu_f, f), getattr(gpu_s, f)), f


@pytest.mark.parametrize("varlen", [False, True])
def test_nvfp4_plain_step_parity(varlen):
    """Steps read the NVFP4 checkpoint: monolith and split give the same bits
    and match the oracle's readout of the decoded checkpoint."""
    spec = _spec(16, num_slots=40, nheads=32, ngroups=4)
    cache = synth.make_cache(spec, 81)
    step = synth.make_step(spec, 21, 8, 82, 8, varlen=varlen, n_padding=2)
    outs = []
    for algo in ("monolith", "split"):
        t = sd.upload_cache(cache, gh.DEV)
        st = sd.upload_step(step, gh.DEV)
        dc = gh.device_cache(spec, t)
        out = gh.out_tensor(step, spec, "bf16")
        gh.run_step(dc, st, step, out, "bf16", algo)
        torch.cuda.synchronize()
        assert int(dc.status.item()) == 0
        outs.append(out)
        gpu = sd.download_cache(spec, t)
        assert np.array_equal(gpu.state, cache.state) and np.array_equal(gpu.recur, cache.recur)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ref, st_ = O.replay_step(cache.copy(), step)
    assert st_ == 0
    got = gh.to_f64(outs[0])
    assert gh.rel_err(got, ref) <= 2e-2, gh.rel_err(got, ref)


def test_nvfp4_fused_empty_windows_equal_flush_then_step():
    """Varlen entries without new tokens, some folding their whole live prefix
    (empty readout window): the fused step gives the GPU's flush-then-step bits."""
    from tests.test_gpu_fused import _with_empty_entries
    spec = _spec(16, num_slots=24, nheads=16, ngroups=2)
    cache = synth.make_cache(spec, 81)
    step = synth.make_step(spec, 11, 4, 82, 6, varlen=True)
    step.pnat[[0, 5, 10]] = [4, 2, 6]
    step.pnat[3] = 0
    step = _with_empty_entries(step, [0, 3, 5, 10])
    k = _fold_counts(step, 83)
    k[[0, 5, 10]] = step.pnat[[0, 5, 10]]
    k[3] = 0
    seed = 87
    print("nvfp4 empty windows Tb", np.diff(step.cu_seqlens), "pnat", step.pnat, "k", k, flush=True)
    out_f, gpu_f, st_f = _run_fused(spec, cache, step, k, seed)
    assert st_f == 0
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    st = sd.upload_step(step, gh.DEV)
    ssu.flush(dc, st["slot_idx"], torch.from_numpy(k).to(gh.DEV), st["A"], sr_seed=seed)
    step2 = synth.StepInputs(**{**step.__dict__, "pnat": (step.pnat - k).astype(np.int32)})
    st2 = sd.upload_step(step2, gh.DEV)
    out_s = gh.out_tensor(step, spec, "bf16")
    gh.run_step(dc, st2, step2, out_s, "bf16", "monolith")
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    gpu_s = sd.download_cache(spec, t)
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    for f in sd.CACHE_FIELDS + ("recur", "gscale", "ring_start"):
        assert np.array_equal(getattr(gpu_f, f), getattr(gpu_s, f)), f
