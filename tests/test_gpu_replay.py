"""GPU parity of the replay step, flush and init against the CPU oracle.

Every test here runs the HIP kernels through the C ABI (libssu.so via the
ctypes binding) and compares element by element with the fp64 oracle on the
same seeded inputs.  Bounds: |err| <= 1e-4 (1 + |ref|) for fp32 state with
fp32 output, <= 2e-2 (1 + |ref|) otherwise; fp8 checkpoints: >= 99.9 % of
codes equal the oracle's, the rest within one code; ring appends of x and B
bit-exact, dt' within 1e-6 (1 + |ref|); untouched memory bit-exact.
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


# Reduced copies of the five workloads: the oracle finishes them in seconds,
# and they still span several workgroups, ragged tails (batch not a multiple
# of the tile), padding entries and ring wraparound.
CASES = {
    "tiny_f32": dict(spec=dict(num_slots=4, nheads=8, ngroups=1, state_dtype="f32"), batch=2, T=1,
                     pnat_max=8, out="f32"),
    "mtp_bf16": dict(spec=dict(num_slots=128, nheads=64, ngroups=8, state_dtype="bf16"), batch=64, T=4,
                     pnat_max=4, out="bf16"),
    "prod_f16": dict(spec=dict(num_slots=80, nheads=128, ngroups=8, state_dtype="f16"), batch=37, T=8,
                     pnat_max=8, out="bf16", n_padding=2),
    "fp8": dict(spec=dict(num_slots=48, nheads=128, ngroups=8, state_dtype="fp8"), batch=33, T=4,
                pnat_max=12, out="bf16"),
    "large_bf16_varlen": dict(spec=dict(num_slots=96, nheads=128, ngroups=8, state_dtype="bf16",
                                        slot_pad=256), batch=41, T=8, pnat_max=8, out="bf16",
                              varlen=True, n_padding=3),
    "bf16_f32out": dict(spec=dict(num_slots=20, nheads=16, ngroups=2, state_dtype="bf16"), batch=9, T=3,
                        pnat_max=13, out="f32"),
    "f32_T16_L32": dict(spec=dict(num_slots=10, nheads=8, ngroups=4, state_dtype="f32", ring_len=32),
                        batch=5, T=16, pnat_max=16, out="f32"),
    "f16_hpg1": dict(spec=dict(num_slots=12, nheads=6, ngroups=6, state_dtype="f16", ring_len=12),
                     batch=7, T=5, pnat_max=7, out="bf16"),
    # 342 x 96 = 32832 (entry, head) pairs, groups of 12 heads: a plain bf16 monolith step runs one head per
    # wave; plain fp8 steps (33 x 128 and 256 x 128 pairs) run in the one-head kernel at any size
    "bf16_per_head": dict(spec=dict(num_slots=400, nheads=96, ngroups=8, state_dtype="bf16"), batch=342, T=4,
                          pnat_max=8, out="bf16", varlen=True, n_padding=3),
    "fp8_per_head": dict(spec=dict(num_slots=300, nheads=128, ngroups=8, state_dtype="fp8"), batch=256, T=4,
                         pnat_max=12, out="bf16", n_padding=2),
    # up to 512 fp8 pairs: one head per wave, one wave per workgroup
    "fp8_small": dict(spec=dict(num_slots=10, nheads=64, ngroups=8, state_dtype="fp8"), batch=6, T=4,
                      pnat_max=12, out="bf16", varlen=True, n_padding=1),
    # 16-bit checkpoints from 1536 pairs (groups of a multiple of 8 heads, rings up to 16): two heads per
    # wave (groups of 16 and of 8); prod_f16, mtp_bf16 and large_bf16_varlen above run there too
    "f16_pair": dict(spec=dict(num_slots=300, nheads=128, ngroups=8, state_dtype="f16"), batch=256, T=8,
                     pnat_max=8, out="bf16", varlen=True, n_padding=3),
    "bf16_pair_hpg8": dict(spec=dict(num_slots=600, nheads=64, ngroups=8, state_dtype="bf16"), batch=512, T=4,
                           pnat_max=4, out="bf16", n_padding=2),
    # 769 to 1535 pairs of a 16-bit checkpoint: the persistent kernel
    "f16_persistent": dict(spec=dict(num_slots=20, nheads=128, ngroups=8, state_dtype="f16"), batch=10, T=8,
                           pnat_max=8, out="bf16", varlen=True, n_padding=1),
    # 800 pairs of fp32: each head's rows in 2 parts (fp32 plain steps split at any size; the split
    # algorithm runs the persistent kernel)
    "f32_mid": dict(spec=dict(num_slots=120, nheads=8, ngroups=2, state_dtype="f32"), batch=100, T=3,
                    pnat_max=10, out="f32", n_padding=4),
    # 16-bit up to 768 pairs: each head's rows split over waves, 2 parts from 257 pairs, 4 parts up to 256
    # (tiny_f32, bf16_f32out, f32_T16_L32 and f16_hpg1 above run in 4 parts)
    "bf16_dsplit2": dict(spec=dict(num_slots=8, nheads=128, ngroups=8, state_dtype="bf16"), batch=4, T=6,
                         pnat_max=8, out="bf16", varlen=True, n_padding=1),
    "f32_dsplit2_L32": dict(spec=dict(num_slots=48, nheads=8, ngroups=2, state_dtype="f32", ring_len=32),
                            batch=40, T=12, pnat_max=20, out="f32", n_padding=2),
    "f16_dsplit4_L24": dict(spec=dict(num_slots=16, nheads=16, ngroups=4, state_dtype="f16", ring_len=24),
                            batch=10, T=5, pnat_max=19, out="bf16", varlen=True, n_padding=1),
}


def _setup(case, seed):
    cfg = CASES[case]
    spec = synth.CacheSpec(**cfg["spec"])
    cache = synth.make_cache(spec, seed)
    step = synth.make_step(spec, cfg["batch"], cfg["T"], seed + 1, cfg["pnat_max"],
                           varlen=cfg.get("varlen", False), n_padding=cfg.get("n_padding", 0))
    return spec, cache, step, cfg["out"]


@pytest.mark.parametrize("algo", ["monolith", "split"])
@pytest.mark.parametrize("case", list(CASES))
def test_replay_step_parity(case, algo):
    spec, cache, step, out_dtype = _setup(case, 1000 + len(case))
    print("case", case, algo, flush=True)
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, out_dtype)
    gh.run_step(dc, st, step, out, out_dtype, algo)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    ref_cache = cache.copy()
    ref, status = O.replay_step(ref_cache, step)
    assert status == 0
    got = gh.to_f64(out)
    err = gh.rel_err(got, ref)
    assert err <= gh.tol_for(spec.state_dtype, out_dtype), "max rel err %g" % err
    gh.check_cache_after_step(spec, cache, sd.download_cache(spec, t), ref_cache)


@pytest.mark.parametrize("case", list(CASES))
def test_monolith_split_bit_exact(case):
    spec, cache, step, out_dtype = _setup(case, 2000 + len(case))
    outs, caches = [], []
    for algo in ("monolith", "split"):
        t = sd.upload_cache(cache, gh.DEV)
        st = sd.upload_step(step, gh.DEV)
        dc = gh.device_cache(spec, t)
        out = gh.out_tensor(step, spec, out_dtype)
        gh.run_step(dc, st, step, out, out_dtype, algo)
        torch.cuda.synchronize()
        outs.append(out.view(torch.uint8).cpu().numpy() if out.dtype != torch.float32
                    else out.view(torch.int32).cpu().numpy())
        caches.append(sd.download_cache(spec, t))
    assert np.array_equal(outs[0], outs[1])
    for f in sd.CACHE_FIELDS:
        assert np.array_equal(getattr(caches[0], f), getattr(caches[1], f)), f


def test_replay_deterministic_and_idempotent():
    spec, cache, step, out_dtype = _setup("prod_f16", 77)
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    res = []
    for rep in range(3):
        for algo in ("split", "monolith"):
            out = gh.out_tensor(step, spec, out_dtype)
            gh.run_step(dc, st, step, out, out_dtype, algo)
            res.append(out.view(torch.int16).cpu().numpy())
    for r in res[1:]:
        assert np.array_equal(r, res[0])


@pytest.mark.parametrize("state_dtype", ["f32", "bf16", "f16", "fp8"])
def test_flush_parity(state_dtype):
    spec = synth.CacheSpec(num_slots=40, nheads=32, ngroups=4, state_dtype=state_dtype)
    cache = synth.make_cache(spec, 31)
    step = synth.make_step(spec, 30, 4, 32, 8)
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, "bf16")
    gh.run_step(dc, st, step, out, "bf16", "monolith")
    ref = cache.copy()
    O.replay_step(ref, step)
    # fold between 0 and pnat + T tokens; include the k = 0 no-op and k = L - 1
    rng = np.random.default_rng(5)
    k = np.array([rng.integers(0, int(p) + 5) for p in step.pnat], np.int32)
    k[0], k[1] = 0, min(int(step.pnat[1]) + 4, spec.ring_len)
    kt = torch.from_numpy(k).to(gh.DEV)
    ssu.flush(dc, st["slot_idx"], kt, st["A"])
    torch.cuda.synchronize()
    assert int(dc.status.item()) == 0
    before_flush = ref.copy()
    assert O.flush(ref, step.slot_idx, k, step.A) == 0
    gpu = sd.download_cache(spec, t)
    assert np.array_equal(gpu.ring_start, ref.ring_start)
    for f in ("x_cache", "B_cache", "dt_cache"):
        assert np.array_equal(getattr(gpu, f), getattr(before_flush, f)) or f == "dt_cache"
    touched = [int(s) for s, kk in zip(step.slot_idx, k) if kk > 0]
    untouched = [s for s in range(spec.num_slots) if s not in touched]
    assert np.array_equal(gpu.state[untouched], before_flush.state[untouched])
    nb = spec.state_bytes()
    assert np.array_equal(gpu.state[:, nb:], before_flush.state[:, nb:])  # canaries
    if state_dtype == "fp8":
        gh.check_state(spec, gpu, ref, before_flush, touched, (step.slot_idx, k, step.A))
    else:
        g = np.stack([O.decode_state(gpu, s) for s in touched])
        r = np.stack([O.decode_state(ref, s) for s in touched])
        tol = 1e-4 if state_dtype == "f32" else 2e-2
        assert gh.rel_err(g, r) <= tol


@pytest.mark.parametrize("state_dtype", ["f32", "bf16", "f16", "fp8"])
@pytest.mark.parametrize("broadcast", [False, True])
def test_init_state_parity(state_dtype, broadcast):
    spec = synth.CacheSpec(num_slots=12, nheads=16, ngroups=2, state_dtype=state_dtype, slot_pad=64)
    cache = synth.make_cache(spec, 41)
    rng = np.random.default_rng(6)
    n = 6
    states = (rng.standard_normal((n, 16, 64, 128)) * 0.2).astype(np.float32)
    states[1, 3, 5, :] = 0.0
    states[2, 0, 0, 7] = 1e-39  # a subnormal-only row element
    ids = np.array([3, 0, 7, 12, 11, 1], np.int32)
    t = sd.upload_cache(cache, gh.DEV)
    dc = gh.device_cache(spec, t)
    st = torch.from_numpy(states).to(gh.DEV)
    ids_t = torch.from_numpy(ids).to(gh.DEV)
    ssu.init_state(dc, st, ids_t, states_batch_stride=0 if broadcast else None)
    torch.cuda.synchronize()
    ref = cache.copy()
    O.init_state(ref, states, ids, states_stride=0 if broadcast else None)
    gpu = sd.download_cache(spec, t)
    assert np.array_equal(gpu.ring_start, ref.ring_start)
    for f in ("x_cache", "B_cache", "dt_cache", "scale"):
        if f == "scale" and state_dtype == "fp8":
            continue
        assert np.array_equal(getattr(gpu, f), getattr(ref, f)), f
    if state_dtype == "fp8":
        frac, dist = gh.fp8_code_agreement(gpu.state, ref.state)
        assert frac >= 0.999 and dist <= 1
        assert np.array_equal(gpu.scale, ref.scale)  # same fp32 division of the same input
    else:
        assert np.array_equal(gpu.state, ref.state)


def test_status_bits_and_padding():
    spec = synth.CacheSpec(num_slots=16, nheads=16, ngroups=2, state_dtype="bf16")
    cache = synth.make_cache(spec, 51)
    step = synth.make_step(spec, 6, 4, 52, 4)
    step.slot_idx[0] = 0                      # padding
    step.slot_idx[1] = spec.num_slots + 3     # out of range: padding
    step.pnat[2] = spec.ring_len - 1          # pnat + T > L
    for algo in ("monolith", "split"):
        t = sd.upload_cache(cache, gh.DEV)
        st = sd.upload_step(step, gh.DEV)
        dc = gh.device_cache(spec, t)
        out = gh.out_tensor(step, spec, "bf16")
        gh.run_step(dc, st, step, out, "bf16", algo)
        torch.cuda.synchronize()
        assert int(dc.status.item()) == ssu.SSU_STATUS_BAD_PNAT
        ref_cache = cache.copy()
        ref, status = O.replay_step(ref_cache, step)
        assert status == 1
        got = gh.to_f64(out)
        assert np.all(got[:12] == 0.0)
        assert gh.rel_err(got, ref) <= 2e-2
        gh.check_cache_after_step(spec, cache, sd.download_cache(spec, t), ref_cache)
    # flush with k out of range and a bad ring_start
    t = sd.upload_cache(cache, gh.DEV)
    t["ring_start"][int(step.slot_idx[4])] = spec.ring_len + 2
    dc = gh.device_cache(spec, t)
    st = sd.upload_step(step, gh.DEV)
    k = torch.tensor([1, 1, 1, spec.ring_len + 1, 2, 0], dtype=torch.int32, device=gh.DEV)
    before = sd.download_cache(spec, t)
    ssu.flush(dc, st["slot_idx"], k, st["A"])
    torch.cuda.synchronize()
    assert int(dc.status.item()) == ssu.SSU_STATUS_BAD_FOLD | ssu.SSU_STATUS_BAD_RING
    after = sd.download_cache(spec, t)
    for b in (3, 4, 5):
        s = int(step.slot_idx[b])
        assert np.array_equal(after.state[s], before.state[s])


@pytest.mark.parametrize("state_dtype", ["bf16", "f16"])
def test_pair_path_empty_entries(state_dtype):
    """Two heads per wave (plain 16-bit steps from 1536 pairs) with varlen
    entries that have no new token, padding entries and the last entry empty:
    bit for bit against the split, and against the oracle."""
    from tests.test_gpu_fused import _with_empty_entries
    spec = synth.CacheSpec(num_slots=300, nheads=128, ngroups=8, state_dtype=state_dtype, slot_pad=256)
    cache = synth.make_cache(spec, 4100)
    step = synth.make_step(spec, 256, 8, 4101, 8, varlen=True, n_padding=4)
    step = _with_empty_entries(step, [0, 17, 100, 255])
    print("pair path empty entries", state_dtype, "Tb", np.diff(step.cu_seqlens)[:20], flush=True)
    outs, caches = [], []
    for algo in ("monolith", "split"):
        t = sd.upload_cache(cache, gh.DEV)
        st = sd.upload_step(step, gh.DEV)
        dc = gh.device_cache(spec, t)
        out = gh.out_tensor(step, spec, "bf16")
        gh.run_step(dc, st, step, out, "bf16", algo)
        torch.cuda.synchronize()
        assert int(dc.status.item()) == 0
        outs.append(out)
        caches.append(sd.download_cache(spec, t))
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    for f in sd.CACHE_FIELDS + ("ring_start",):
        assert np.array_equal(getattr(caches[0], f), getattr(caches[1], f)), f
    ref_cache = cache.copy()
    ref, status = O.replay_step(ref_cache, step)
    assert status == 0
    assert gh.rel_err(gh.to_f64(outs[0]), ref) <= gh.tol_for(state_dtype, "bf16")
    gh.check_cache_after_step(spec, cache, caches[0], ref_cache)


# every replay path: (case, algo, fold) -> the kernel the step runs in
BAD_RING_PATHS = [
    ("tiny_f32", "monolith", False),        # head rows in 4 parts
    ("bf16_dsplit2", "monolith", False),    # head rows in 2 parts
    ("f16_persistent", "monolith", False),  # persistent kernel
    ("f16_pair", "monolith", False),        # two heads per wave
    ("f16_pair", "split", False),           # C.B precompute + persistent kernel
    ("fp8_per_head", "monolith", False),    # one head per wave, nothing folded
    ("fp8", "split", False),                # C.B precompute + persistent kernel, fp8 tile
    ("fp8_per_head", "auto", True),         # fused flush-in-step
]


@pytest.mark.parametrize("case,algo,fold", BAD_RING_PATHS)
def test_bad_ring_start_each_path(case, algo, fold):
    """An entry whose slot's ring_start lies outside [0, L) (one past the
    end, one negative) is skipped on every path: its output rows are zero,
    its rings, checkpoint and ring_start stay as they were, and the status
    word says SSU_STATUS_BAD_RING; every other entry matches the oracle,
    which skips such entries the same way."""
    spec, cache, step, out_dtype = _setup(case, 4200 + len(case))
    live = [b for b in range(step.batch) if 0 < step.slot_idx[b] < spec.num_slots]
    bad = [live[0], live[len(live) // 2]]
    cache.ring_start[int(step.slot_idx[bad[0]])] = spec.ring_len + 3
    cache.ring_start[int(step.slot_idx[bad[1]])] = -1
    print("case", case, algo, "fold" if fold else "", "bad entries", bad, flush=True)
    k = None
    if fold:
        k = np.minimum(step.pnat, 1).astype(np.int32)
    t = sd.upload_cache(cache, gh.DEV)
    st = sd.upload_step(step, gh.DEV)
    dc = gh.device_cache(spec, t)
    out = gh.out_tensor(step, spec, out_dtype)
    if fold:
        kt = torch.from_numpy(k).to(gh.DEV)
        desc = ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                                  st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, out_dtype,
                                  None, algo, num_fold=kt)
        ssu.replay_step(dc, desc)
    else:
        gh.run_step(dc, st, step, out, out_dtype, algo)
    torch.cuda.synchronize()
    assert int(dc.status.item()) == ssu.SSU_STATUS_BAD_RING
    gpu = sd.download_cache(spec, t)
    ref_cache = cache.copy()
    ref, status = O.replay_step(ref_cache, step, num_fold=k) if fold else O.replay_step(ref_cache, step)
    assert status == ssu.SSU_STATUS_BAD_RING
    got = gh.to_f64(out)
    cu = step.cu_seqlens if step.cu_seqlens is not None else np.arange(step.batch + 1) * step.T
    for b in bad:
        assert np.all(got[cu[b]:cu[b + 1]] == 0.0)
        s = int(step.slot_idx[b])
        for f in sd.CACHE_FIELDS:
            assert np.array_equal(getattr(gpu, f)[s], getattr(cache, f)[s]), f
        assert gpu.ring_start[s] == cache.ring_start[s]
    if fold:
        gh.check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, out_dtype)
    else:
        assert gh.rel_err(got, ref) <= gh.tol_for(spec.state_dtype, out_dtype)
        gh.check_cache_after_step(spec, cache, gpu, ref_cache)
    assert np.array_equal(gpu.ring_start, ref_cache.ring_start)
