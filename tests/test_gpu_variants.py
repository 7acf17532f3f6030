"""GPU parity of the step variants: the z-gated output and dt' without
softplus, alone, together, with the split and with a fused flush.

Same bounds as the reduced parity tests; monolith and split stay
bit-identical with the variants on.
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
from tests.test_gpu_replay import CASES


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _setup(case, seed, with_z, dt_softplus):
    cfg = CASES[case]
    spec = synth.CacheSpec(**cfg["spec"])
    cache = synth.make_cache(spec, seed)
    step = synth.make_step(spec, cfg["batch"], cfg["T"], seed + 1, cfg["pnat_max"],
                           varlen=cfg.get("varlen", False), n_padding=cfg.get("n_padding", 0),
                           with_z=with_z, dt_softplus=dt_softplus)
    return spec, cache, step, cfg["out"]


def _run(spec, cache, step, out_dtype, algo, k=None):
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
                              algo, num_fold=kt, z=st["z"], dt_softplus=step.dt_softplus)
    ssu.replay_step(dc, desc)
    torch.cuda.synchronize()
    return out, sd.download_cache(spec, t), int(dc.status.item())


VARIANTS = [(True, True), (False, False), (True, False)]


@pytest.mark.parametrize("with_z,dt_softplus", VARIANTS)
@pytest.mark.parametrize("case", ["tiny_f32", "mtp_bf16", "prod_f16", "fp8", "large_bf16_varlen", "bf16_f32out",
                                  "f32_T16_L32"])
def test_variant_parity(case, with_z, dt_softplus):
    seed = 6000 + len(case) + 10 * with_z + 20 * dt_softplus
    spec, cache, step, out_dtype = _setup(case, seed, with_z, dt_softplus)
    print("case", case, "z", with_z, "softplus", dt_softplus, flush=True)
    outs = []
    for algo in ("monolith", "split"):
        out, gpu, status = _run(spec, cache, step, out_dtype, algo)
        assert status == 0
        outs.append(out)
        ref_cache = cache.copy()
        ref, st = O.replay_step(ref_cache, step)
        assert st == 0
        err = gh.rel_err(gh.to_f64(out), ref)
        assert err <= gh.tol_for(spec.state_dtype, out_dtype), "%s max rel err %g" % (algo, err)
        gh.check_cache_after_step(spec, cache, gpu, ref_cache)
    view = torch.int32 if outs[0].dtype == torch.float32 else torch.int16
    assert torch.equal(outs[0].view(view), outs[1].view(view))


@pytest.mark.parametrize("with_z,dt_softplus", [(True, True), (True, False)])
@pytest.mark.parametrize("case", ["bf16_per_head", "fp8_per_head"])
def test_variant_parity_one_head_per_wave(case, with_z, dt_softplus):
    """At 256 x 128 (entry, head) pairs a plain bf16 / fp8 monolith step runs
    one head per wave: the variants there, against the oracle and bit for bit
    against the split (persistent) kernel."""
    test_variant_parity(case, with_z, dt_softplus)


@pytest.mark.parametrize("case", ["fp8", "prod_f16"])
def test_variants_with_fused_flush(case):
    spec, cache, step, out_dtype = _setup(case, 6100 + len(case), True, False)
    rng = np.random.default_rng(3)
    k = np.array([rng.integers(0, int(p) + 1) for p in step.pnat], np.int32)
    out, gpu, status = _run(spec, cache, step, out_dtype, "auto", k)
    assert status == 0
    ref_cache = cache.copy()
    ref, st = O.replay_step(ref_cache, step, num_fold=k)
    assert st == 0
    gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, out_dtype)
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
    touched = sorted({int(s) for s, kk in zip(step.slot_idx, k) if kk > 0 and 0 < s < spec.num_slots})
    gh.check_state(spec, gpu, ref_cache, cache, touched, (step.slot_idx, k, step.A))
