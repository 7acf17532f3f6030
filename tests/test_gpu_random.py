"""GPU parity over random shapes inside the documented limits.

The fixed cases elsewhere pick shapes by the kernel they reach.  Here 64
seeded draws pick every dimension at random inside what include/ssu.h
allows, so that the dispatch meets combinations nobody chose:
  - state dtype (fp32, bf16, fp16, fp8);
  - groups and heads per group (1 to 16);
  - ring length 1 to 32, then T up to min(16, L) and pnat up to L - T;
  - batch (1 to 48; half of the bf16 and fp16 draws take 128 heads in groups
    of 16 and enough entries for the two-heads-per-wave range);
  - varlen, padding entries and slot padding;
  - output dtype, the z gate and dt' without softplus.
Each draw runs the plain step (monolith and split, bit for bit with each
other), the fused flush-in-step and a flush of the same k, against the
oracle at the same bounds as the fixed cases.  32 more draws do the same with separate checkpoints (an
fp8 or NVFP4 read checkpoint beside the FP16 recurrence checkpoint, folded
with stochastic rounding under a drawn seed), whose folds are checked as the
fixed separate-checkpoint cases check theirs.  24 draws run ssu_init_state
over random shapes and id lists in every checkpoint form.  The draw is
printed before its GPU work.
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

N_DRAWS = 64
N_SEPARATE = 32


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw(i):
    rng = np.random.default_rng(90000 + i)
    state = ["f32", "bf16", "f16", "fp8"][i % 4]
    G = int(rng.choice([1, 2, 3, 4, 8]))
    hpg = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    L = int(rng.integers(1, 33))
    T = int(rng.integers(1, min(16, L) + 1))
    pnat_max = int(rng.integers(0, L - T + 1))
    H = G * hpg
    if i % 8 in (5, 6):  # half of the bf16 and fp16 draws: the two-heads-per-wave range
        G, hpg, L = 8, 16, min(L, 16)
        H, T = 128, min(T, L)
        pnat_max = min(pnat_max, L - T)
        batch = int(rng.integers(12, 20))
    else:
        batch = int(rng.integers(1, 49))
    n_padding = int(rng.integers(0, batch // 4 + 1))
    spec = dict(num_slots=batch + int(rng.integers(1, 8)), nheads=H, ngroups=G, state_dtype=state, ring_len=L,
                slot_pad=int(rng.choice([0, 256])))
    return dict(spec=spec, batch=batch, T=T, pnat_max=pnat_max, varlen=bool(rng.integers(0, 2)),
                n_padding=n_padding, out="f32" if (state == "f32" or rng.integers(0, 4) == 0) else "bf16",
                with_z=bool(rng.integers(0, 4) == 0), dt_softplus=bool(rng.integers(0, 4) != 0))


def draw_separate(i):
    """A draw with separate checkpoints: fp8 or NVFP4 read checkpoint."""
    rng = np.random.default_rng(95000 + i)
    state = ["fp8", "nvfp4"][i % 2]
    G = int(rng.choice([1, 2, 3, 4, 8]))
    hpg = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    L = int(rng.integers(1, 33))
    T = int(rng.integers(1, min(16, L) + 1))
    batch = int(rng.integers(1, 41))
    spec = dict(num_slots=batch + int(rng.integers(1, 8)), nheads=G * hpg, ngroups=G, state_dtype=state,
                ring_len=L, slot_pad=int(rng.choice([0, 256])), separate=True)
    return dict(spec=spec, batch=batch, T=T, pnat_max=int(rng.integers(0, L - T + 1)),
                varlen=bool(rng.integers(0, 2)), n_padding=int(rng.integers(0, batch // 4 + 1)),
                out="f32" if rng.integers(0, 4) == 0 else "bf16", with_z=bool(rng.integers(0, 4) == 0),
                dt_softplus=bool(rng.integers(0, 4) != 0), sr_seed=int(rng.integers(0, 2 ** 63)))


def _run(spec, cache, step, out_dtype, algo, k=None, sr_seed=0):
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, out_dtype)
    ws = None
    if algo == "split":
        ws = torch.empty(max(ssu.workspace_size(dc, step.batch, step.T) // 4, 1), dtype=torch.float32,
                         device=gh.DEV)
    kt = None if k is None else torch.from_numpy(k).to(gh.DEV)
    desc = ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                              st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, out_dtype, ws,
                              algo, num_fold=kt, z=st["z"], dt_softplus=step.dt_softplus, sr_seed=sr_seed)
    ssu.replay_step(dc, desc)
    torch.cuda.synchronize()
    return out, sd.download_cache(spec, t), int(dc.status.item())


@pytest.mark.parametrize("i", range(N_DRAWS))
def test_random_shape_parity(i):
    check_draw(draw(i), i)


@pytest.mark.parametrize("i", range(N_SEPARATE))
def test_random_shape_separate_parity(i):
    check_draw(draw_separate(i), 1000 + i)


def check_draw(d, i):
    spec = synth.CacheSpec(**d["spec"])
    seed = d.get("sr_seed", 0)
    print("draw", i, {k: v for k, v in d.items() if k != "spec"}, d["spec"], flush=True)
    cache = synth.make_cache(spec, 91000 + i)
    step = synth.make_step(spec, d["batch"], d["T"], 92000 + i, d["pnat_max"], varlen=d["varlen"],
                           n_padding=d["n_padding"], with_z=d["with_z"], dt_softplus=d["dt_softplus"])
    out_dtype = d["out"]
    tol = gh.tol_for(spec.state_dtype, out_dtype)

    # plain step: monolith and split against the oracle, and bit for bit with each other
    ref_cache = cache.copy()
    ref, status = O.replay_step(ref_cache, step)
    assert status == 0
    outs = []
    for algo in ("monolith", "split"):
        out, gpu, status = _run(spec, cache, step, out_dtype, algo)
        assert status == 0, algo
        err = gh.rel_err(gh.to_f64(out), ref)
        assert err <= tol, "%s: max rel err %g" % (algo, err)
        gh.check_cache_after_step(spec, cache, gpu, ref_cache)
        if spec.separate:  # a plain step leaves the recurrence checkpoint and the slot scales alone
            assert np.array_equal(gpu.recur, cache.recur)
            assert np.array_equal(gpu.gscale, cache.gscale)
        outs.append(out)
    view = torch.int32 if outs[0].dtype == torch.float32 else torch.int16
    assert torch.equal(outs[0].view(view), outs[1].view(view))

    # fused flush-in-step with k ~ U{0..pnat}
    rng = np.random.default_rng(93000 + i)
    k = np.array([rng.integers(0, int(p) + 1) for p in step.pnat], np.int32)
    out, gpu, status = _run(spec, cache, step, out_dtype, "auto", k, seed)
    assert status == 0
    ref_cache = cache.copy()
    ref, status = O.replay_step(ref_cache, step, num_fold=k, seed=seed)
    assert status == 0
    gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, out_dtype)
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    assert np.array_equal(gpu.x_cache, ref_cache.x_cache)
    assert np.array_equal(gpu.B_cache, ref_cache.B_cache)
    nb = spec.dt_bytes()
    gd = gpu.dt_cache[:, :nb].view(np.float32).astype(np.float64)
    rd = ref_cache.dt_cache[:, :nb].view(np.float32).astype(np.float64)
    assert gh.rel_err(gd, rd) <= 1e-6
    touched = sorted({int(s) for s, kk in zip(step.slot_idx, k) if kk > 0 and 0 < s < spec.num_slots})
    gh.check_state(spec, gpu, ref_cache, cache, touched, (step.slot_idx, k, step.A))
    if spec.separate:
        gh.check_recur(spec, gpu, cache, step.slot_idx, k, step.A, seed)

    # the same k as a flush on its own
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    st = sd.upload_step(step, gh.DEV)
    ssu.flush(dc, st["slot_idx"], torch.from_numpy(k).to(gh.DEV), st["A"], sr_seed=seed)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    gpu = sd.download_cache(spec, t)
    ref_cache = cache.copy()
    assert O.flush(ref_cache, step.slot_idx, k, step.A, seed) == 0
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    for f in ("x_cache", "B_cache", "dt_cache"):
        assert np.array_equal(getattr(gpu, f), getattr(cache, f)), f
    gh.check_state(spec, gpu, ref_cache, cache, touched, (step.slot_idx, k, step.A))
    if spec.separate:
        gh.check_recur(spec, gpu, cache, step.slot_idx, k, step.A, seed)


# init over random shapes: (state dtype, separate checkpoints)
INIT_FORMS = [("f32", False), ("bf16", False), ("f16", False), ("fp8", False), ("fp8", True), ("nvfp4", True)]
N_INIT = 24


@pytest.mark.parametrize("i", range(N_INIT))
def test_random_init_parity(i):
    """ssu_init_state over random shapes, id lists (unique valid ids among
    padding and out-of-range ones), row magnitudes (zero rows among them) and
    batch strides (a stride-0 broadcast now and then): rings cleared and
    ring starts zeroed bit for bit; 32- and 16-bit checkpoints bit for bit;
    fp8 codes >= 99.9 % equal and otherwise one code apart with the row scales
    bit for bit; the FP16 recurrence checkpoint bit for bit (same Philox
    bits); NVFP4 slot and block scales bit for bit and >= 99.99 % of the
    decoded values equal."""
    rng = np.random.default_rng(97000 + i)
    state, sep = INIT_FORMS[i % len(INIT_FORMS)]
    G = int(rng.choice([1, 2, 3, 4, 8]))
    H = G * int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    num_slots = int(rng.integers(2, 40))
    spec = synth.CacheSpec(num_slots=num_slots, nheads=H, ngroups=G, state_dtype=state, separate=sep,
                           ring_len=int(rng.integers(1, 33)), slot_pad=int(rng.choice([0, 64, 256])))
    valid = rng.permutation(np.arange(1, num_slots))[:int(rng.integers(1, num_slots))]
    invalid = rng.choice([0, -1, num_slots, num_slots + 5], int(rng.integers(0, 4)))
    ids = rng.permutation(np.concatenate([valid, invalid])).astype(np.int32)
    n = ids.size
    states = (rng.standard_normal((n, H, 64, 128)) * rng.uniform(0.01, 3.0, (n, H, 64, 1))).astype(np.float32)
    states[rng.random((n, H, 64)) < 0.02] = 0.0
    broadcast = bool(rng.integers(0, 3) == 0)
    seed = int(rng.integers(0, 2 ** 63))
    print("init draw", i, state, "separate", sep, "H", H, "G", G, "L", spec.ring_len, "slots", num_slots, "n", n,
          "broadcast", broadcast, flush=True)
    cache = synth.make_cache(spec, 98000 + i)
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    ssu.init_state(dc, torch.from_numpy(states).to(gh.DEV), torch.from_numpy(ids).to(gh.DEV),
                   states_batch_stride=0 if broadcast else None, sr_seed=seed)
    torch.cuda.synchronize()
    ref = cache.copy()
    O.init_state(ref, states, ids, states_stride=0 if broadcast else None, seed=seed)
    gpu = sd.download_cache(spec, t)
    for f in ("x_cache", "B_cache", "dt_cache", "ring_start"):
        assert np.array_equal(getattr(gpu, f), getattr(ref, f)), f
    others = np.setdiff1d(np.arange(num_slots), valid)  # slot 0 and every slot not named: untouched
    for f in ("state", "scale", "recur", "gscale"):
        a = getattr(gpu, f)
        if a is not None:
            assert np.array_equal(a[others], getattr(cache, f)[others]), f
    if sep:
        assert np.array_equal(gpu.recur, ref.recur)
    if state == "nvfp4":
        assert np.array_equal(gpu.gscale, ref.gscale)
        assert np.array_equal(gpu.scale, ref.scale)
        for sl in valid:
            g, r = O.decode_state(gpu, int(sl)), O.decode_state(ref, int(sl))
            assert np.mean(g == r) >= 0.9999, int(sl)
    elif state == "fp8":
        assert np.array_equal(gpu.scale, ref.scale)
        nb = spec.state_bytes()  # the codes of the named slots only
        frac, dist = gh.fp8_code_agreement(gpu.state[valid, :nb], ref.state[valid, :nb])
        assert frac >= 0.999 and dist <= 1, (frac, dist)
        assert np.array_equal(gpu.state[:, nb:], ref.state[:, nb:])  # slot padding
    else:
        assert np.array_equal(gpu.state, ref.state)
