"""Parity at the benchmark's full sizes, in the launch configurations the
benchmark times, on every entry.

Each case draws a full-size cache on the GPU (the benchmark's value laws),
keeps a device copy of it, runs the step (and flush) on every entry through
the C ABI, and checks:
  - every slot the call does not own, and the padding of every slot page,
    bit for bit against the copy (compared on the device);
  - every entry against the fp64 oracle run on exactly those slots: outputs,
    ring appends, ring_start and, where a flush ran, the re-encoded
    checkpoints (bounds as in the reduced parity tests; a fused step's
    outputs also against the oracle's plain step on the GPU's own post-fold
    checkpoint at the plain bound).
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


# (workload, algo): the five benchmark workloads at their full sizes
FULL = {
    "tiny_b2": dict(nheads=8, ngroups=1, state="f32", batch=2, slots=4, T=1, pnat_max=8, out="f32"),
    "mtp_b64": dict(nheads=64, ngroups=8, state="bf16", batch=64, slots=128, T=4, pnat_max=4, out="bf16"),
    # production sizes at the small end: 4 (rows of each head in parts), 8 (persistent kernel), 32 (two heads
    # per wave)
    "prod_b4": dict(nheads=128, ngroups=8, state="f16", batch=4, slots=9, T=8, pnat_max=8, out="bf16"),
    "prod_b8": dict(nheads=128, ngroups=8, state="f16", batch=8, slots=17, T=8, pnat_max=8, out="bf16"),
    "prod_b32": dict(nheads=128, ngroups=8, state="f16", batch=32, slots=65, T=8, pnat_max=8, out="bf16"),
    "prod_b256": dict(nheads=128, ngroups=8, state="f16", batch=256, slots=513, T=8, pnat_max=8, out="bf16"),
    "prod_b512": dict(nheads=128, ngroups=8, state="f16", batch=512, slots=1025, T=8, pnat_max=8, out="bf16"),
    "fp8_b256": dict(nheads=128, ngroups=8, state="fp8", batch=256, slots=513, T=4, pnat_max=0, out="bf16",
                     flush=(1, 4)),
    # separate checkpoints: an FP16 recurrence checkpoint beside the read checkpoint
    "fp8sep_b256": dict(nheads=128, ngroups=8, state="fp8", batch=256, slots=513, T=4, pnat_max=0, out="bf16",
                        flush=(1, 4), sep=True),
    "nvfp4_b256": dict(nheads=128, ngroups=8, state="nvfp4", batch=256, slots=513, T=4, pnat_max=0,
                       out="bf16", flush=(1, 4), sep=True),
    "large_b1024": dict(nheads=128, ngroups=8, state="bf16", batch=1024, slots=2048, T=8, pnat_max=8,
                        out="bf16", varlen=True, pad=256),
}
RUNS = [("tiny_b2", "monolith"), ("mtp_b64", "monolith"), ("mtp_b64", "split"), ("prod_b4", "monolith"),
        ("prod_b4", "split"), ("prod_b8", "monolith"), ("prod_b32", "monolith"), ("prod_b256", "monolith"),
        ("prod_b256", "split"), ("prod_b512", "monolith"), ("fp8_b256", "fused"), ("fp8_b256", "separate"),
        ("fp8sep_b256", "fused"), ("nvfp4_b256", "fused"), ("nvfp4_b256", "separate"),
        ("large_b1024", "monolith")]


def _packed_bytes(spec):
    """Packed bytes of each per-slot tensor (the rest of a slot page is padding)."""
    d = {"state": spec.state_bytes(), "scale": spec.scale_bytes() if spec.state_dtype in ("fp8", "nvfp4") else 0,
         "x_cache": spec.x_bytes(), "B_cache": spec.B_bytes(), "dt_cache": spec.dt_bytes()}
    if spec.separate:
        d["recur"] = spec.recur_bytes()
    if spec.state_dtype == "nvfp4":
        d["gscale"] = spec.gscale_bytes()
    return d


def _check_untouched_on_device(spec, t, snap, slots):
    """Slots the call does not own and every slot page's padding: bit for bit."""
    owned = torch.zeros(spec.num_slots, dtype=torch.bool, device=gh.DEV)
    owned[torch.from_numpy(np.asarray(slots, np.int64)).to(gh.DEV)] = True
    for f, nb in _packed_bytes(spec).items():
        a, b = t[f], snap[f]
        assert torch.equal(a[~owned], b[~owned]), "%s changed outside the call's slots" % f
        assert torch.equal(a[:, nb:], b[:, nb:]), "%s slot padding changed" % f
    assert torch.equal(t["ring_start"][~owned], snap["ring_start"][~owned])


@pytest.mark.parametrize("name,algo", RUNS)
def test_full_size(name, algo):
    cfg = FULL[name]
    seed = 9000 + len(name) * 7 + len(algo)
    print("case", name, algo, flush=True)
    spec = synth.CacheSpec(num_slots=cfg["slots"], nheads=cfg["nheads"], ngroups=cfg["ngroups"],
                           state_dtype=cfg["state"], slot_pad=cfg.get("pad", 0), separate=cfg.get("sep", False))
    sr_seed = 0x5A5A0000 + seed
    t = sd.make_cache_device(spec, seed, gh.DEV)
    snap = {f: (None if v is None else v.clone()) for f, v in t.items()}
    rng = np.random.default_rng(seed)
    B = cfg["batch"]
    slots = np.sort(rng.choice(np.arange(1, spec.num_slots), B, replace=False)).astype(np.int32)
    step = synth.make_step(spec, B, cfg["T"], seed + 1, cfg["pnat_max"], varlen=cfg.get("varlen", False),
                           slots=slots, pnat_fixed=0 if cfg["pnat_max"] == 0 else None)
    k = None
    if "flush" in cfg:
        k = synth.flush_counts(B, cfg["flush"][0], cfg["flush"][1], seed + 2)
        if algo == "fused":
            step.pnat[:] = k  # the previous step's accepted tokens, folded first

    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, cfg["out"])
    kt = None if k is None else torch.from_numpy(k).to(gh.DEV)
    if algo == "fused":
        desc = ssu.make_step_desc(B, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"], st["B"],
                                  st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, cfg["out"], None,
                                  "auto", num_fold=kt, sr_seed=sr_seed)
        ssu.replay_step(dc, desc)
    else:
        gh.run_step(dc, st, step, out, cfg["out"], "split" if algo == "split" else "monolith")
        if algo == "separate":
            ssu.flush(dc, st["slot_idx"], kt, st["A"], sr_seed=sr_seed)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    _check_untouched_on_device(spec, t, snap, slots)

    # every entry against the oracle, on the call's own slots (renumbered 1..B)
    entries = list(range(B))
    before, smap = sd.download_subset(spec, snap, [int(slots[b]) for b in entries])
    after, _ = sd.download_subset(spec, t, [int(slots[b]) for b in entries])
    del snap
    sub = sd.subset_step(step, entries, smap)
    ref_cache = before.copy()
    ks = None if k is None else k[entries].astype(np.int32)
    if algo == "fused":
        ref, status = O.replay_step(ref_cache, sub, num_fold=ks, seed=sr_seed)
    else:
        ref, status = O.replay_step(ref_cache, sub)
        if algo == "separate":
            mid = ref_cache.copy()  # the state the flush folds from (the step leaves checkpoints alone)
            assert O.flush(ref_cache, sub.slot_idx, ks, sub.A, sr_seed) == 0
    assert status == 0

    if algo == "fused":
        err = gh.check_fused_outputs(after.spec, sub, ks, out, after, ref, ref_cache, cfg["out"])
        print("fused readout rel err vs the oracle on the GPU checkpoint %.3g" % err, flush=True)
    else:
        got = gh.to_f64(out)
        err = gh.rel_err(got, ref)
        assert err <= gh.tol_for(spec.state_dtype, cfg["out"]), err

    assert np.array_equal(after.ring_start, ref_cache.ring_start)
    assert np.array_equal(after.x_cache, ref_cache.x_cache)
    assert np.array_equal(after.B_cache, ref_cache.B_cache)
    nb = spec.dt_bytes()
    assert np.array_equal(after.dt_cache[:, nb:], ref_cache.dt_cache[:, nb:])
    g = after.dt_cache[:, :nb].view(np.float32).astype(np.float64)
    r = ref_cache.dt_cache[:, :nb].view(np.float32).astype(np.float64)
    assert gh.rel_err(g, r) <= 1e-6
    touched = [i + 1 for i in entries if k is not None and k[i] > 0]
    fold = None if ks is None else (sub.slot_idx, ks, sub.A)
    src = mid if algo == "separate" else before
    # the stochastic-rounding brackets and the NVFP4 value bounds on 32 folded
    # slots that hold every fold count (the other checks cover every entry)
    only = None
    if k is not None:
        by_k = {}
        for i in entries:
            if k[i] > 0:
                by_k.setdefault(int(k[i]), []).append(i + 1)
        only = {v[0] for v in by_k.values()}
        rest = [s_ for s_ in touched if s_ not in only]
        only |= set(np.random.default_rng(seed + 3).choice(rest, max(0, min(32 - len(only), len(rest))),
                                                          replace=False).tolist())
    if k is None:
        assert np.array_equal(after.state, before.state)
        assert np.array_equal(after.scale, before.scale)
    else:
        gh.check_state(after.spec, after, ref_cache, src, touched, fold, only=only)
    if spec.separate:  # the recurrence checkpoints, with the random bits of the slots the GPU folded
        bits_slot = {i + 1: int(slots[b]) for i, b in enumerate(entries)}
        gh.check_recur(after.spec, after, src, *fold, sr_seed, bits_slot=bits_slot, only=only)
