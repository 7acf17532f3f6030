"""ssu_replay_step_noalloc through the C ABI: the step for callers that
cannot allocate, whose SPLIT scratch is the library's own device array.

Checked against ssu_replay_step with a caller workspace, bit for bit (outputs
and every cache byte), on two calls in a row on the same GPU with the second
one smaller, and against the oracle at the parity bound; a step whose scratch
would not fit the array is refused before any launch; a step that runs the
monolith (no scratch) gives the same bits as ssu_replay_step.
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


def _run(spec, cache, step, algo, noalloc):
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, "bf16")
    ws = None
    if algo == "split" and not noalloc:
        ws = torch.empty(max(ssu.workspace_size(dc, step.batch, step.T) // 4, 1), dtype=torch.float32,
                         device=gh.DEV)
    desc = ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                              st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, "bf16", ws, algo)
    stream = torch.cuda.current_stream().cuda_stream
    fn = ssu.ssu_replay_step_noalloc if noalloc else ssu.ssu_replay_step
    rc = fn(dc.desc(), desc, stream)
    assert rc == 0, ssu.ssu_last_error()
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    return out, sd.download_cache(spec, t)


CALLS = [  # two calls in a row, the second with a smaller input
    dict(num_slots=80, nheads=32, ngroups=4, state_dtype="f16", batch=61, T=8, pnat_max=8, varlen=False),
    dict(num_slots=80, nheads=32, ngroups=4, state_dtype="f16", batch=9, T=3, pnat_max=5, varlen=True),
]


@pytest.mark.parametrize("algo", ["split", "auto"])
def test_noalloc_matches_replay_step(algo):
    for i, c in enumerate(CALLS):
        spec = synth.CacheSpec(num_slots=c["num_slots"], nheads=c["nheads"], ngroups=c["ngroups"],
                               state_dtype=c["state_dtype"])
        cache = synth.make_cache(spec, 700 + i)
        step = synth.make_step(spec, c["batch"], c["T"], 710 + i, c["pnat_max"], varlen=c["varlen"], n_padding=2)
        print("noalloc call", i, algo, "batch", step.batch, "T", step.T, flush=True)
        out_n, cache_n = _run(spec, cache, step, algo, noalloc=True)
        out_w, cache_w = _run(spec, cache, step, algo, noalloc=False)
        assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16))
        for f in sd.CACHE_FIELDS + ("ring_start",):
            assert np.array_equal(getattr(cache_n, f), getattr(cache_w, f)), f
        ref_cache = cache.copy()
        ref, st = O.replay_step(ref_cache, step)
        assert st == 0
        assert gh.rel_err(gh.to_f64(out_n), ref) <= gh.tol_for(spec.state_dtype, "bf16")
        gh.check_cache_after_step(spec, cache, cache_n, ref_cache)


def _padding_step(spec, batch, T):
    """Device inputs of a step whose entries are all padding (slot 0), every
    buffer at its full size."""
    H, G, rows = spec.nheads, spec.ngroups, batch * T
    z = lambda *shape, dt=torch.int16: torch.zeros(shape, dtype=dt, device=gh.DEV)
    ids = z(batch, dt=torch.int32)
    t = dict(slot_idx=ids, pnat=ids, x=z(rows, H, 64), B=z(rows, G, 128), C=z(rows, G, 128),
             dt=z(rows, H, dt=torch.float32), A=z(H, dt=torch.float32), D=z(H, dt=torch.float32),
             dt_bias=z(H, dt=torch.float32), out=z(rows, H, 64))
    return t, ssu.make_step_desc(batch, T, t["slot_idx"], t["pnat"], None, t["x"], t["B"], t["C"], t["dt"],
                                 t["A"], t["D"], t["dt_bias"], t["out"], "bf16", None, "split")


def test_noalloc_refuses_a_step_past_its_scratch():
    """batch * groups * T * 128 bytes above the array: SSU_ERR_WORKSPACE
    before any launch (the buffers are full size all the same)."""
    spec = synth.CacheSpec(num_slots=4, nheads=16, ngroups=8, state_dtype="bf16")
    cache = synth.make_cache(spec, 3)
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    T = 8
    batch = ssu.SSU_NOALLOC_SCRATCH_BYTES // (spec.ngroups * T * 32 * 4) + 1  # one entry too many
    inputs, desc = _padding_step(spec, batch, T)
    inputs["out"].fill_(7)
    rc = ssu.ssu_replay_step_noalloc(dc.desc(), desc, torch.cuda.current_stream().cuda_stream)
    assert rc == ssu.SSU_ERR_WORKSPACE
    assert "SSU_NOALLOC_SCRATCH_BYTES" in ssu.ssu_last_error()
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    assert bool(torch.all(inputs["out"] == 7))  # nothing ran
    # exactly the array: accepted (all entries padding: zero output rows)
    inputs, desc = _padding_step(spec, batch - 1, T)
    inputs["out"].fill_(7)
    rc = ssu.ssu_replay_step_noalloc(dc.desc(), desc, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, ssu.ssu_last_error()
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    assert torch.count_nonzero(inputs["out"]) == 0
