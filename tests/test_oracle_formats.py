"""Pins of the oracle's number formats, softplus and init against library routines.

The checkpoint encodings are fixed by the vLLM "Add separate CuTeDSL ReplaySSM
checkpoints" page (Claims: FP8 read checkpoints use nearest encoding with
FP32 row scales) and the replayssm_cutedsl page (a zero scale is replaced by
1).  The oracle writes its encoders from the format definitions; here they are
checked against PyTorch's CPU casts (round to nearest even) and a brute-force
nearest-value search.
"""
import numpy as np
import pytest
import torch

import synth
from tests import oracle_refs as R


def _torch_e4m3(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(v32, -448, 448).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _e4m3_probe_values():
    """Every e4m3 value and midpoint, each +-4 fp32 ulps, plus random values."""
    vals = R.e4m3_to_f64(np.arange(0, 127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    base = np.concatenate([vals, mids, [448.0, 460.0, 464.0, 470.0, 1e4]]).astype(np.float32)
    steps = np.arange(-4, 5, dtype=np.int32)
    near = (base.view(np.int32)[:, None] + steps[None, :]).reshape(-1).view(np.float32)
    near = near[np.isfinite(near) & (near >= 0)]
    rng = np.random.default_rng(1)
    rnd = np.concatenate([rng.uniform(0, 500, 200000), np.exp(rng.uniform(-16, 6, 200000))])
    allv = np.concatenate([near, rnd.astype(np.float32)])
    return np.concatenate([allv, -allv]).astype(np.float32)


def test_e4m3_decoder_all_codes(oracle):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_value(codes)
    ref = R.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[1] == 2.0 ** -9


def test_e4m3_encoder_vs_torch(oracle):
    v = _e4m3_probe_values()
    got = oracle.enc_e4m3(v.astype(np.float64))
    ref = _torch_e4m3(v)
    # +-0 both encode zero magnitude
    same = (got == ref) | (((got & 0x7F) == 0) & ((ref & 0x7F) == 0))
    assert same.all(), v[~same][:10]


def test_e4m3_encoder_vs_bruteforce(oracle):
    """Nearest of the 127 finite non-negative values by linear search; ties go
    to the even code."""
    vals = R.e4m3_to_f64(np.arange(0, 127, dtype=np.uint8))
    v = np.abs(_e4m3_probe_values()[:20000].astype(np.float64))
    v = np.minimum(v, 448.0)
    d = np.abs(v[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    code = []
    for c in cand:
        idx = np.flatnonzero(c)
        code.append(idx[0] if len(idx) == 1 else idx[idx % 2 == 0][0])
    code = np.array(code)
    got = oracle.enc_e4m3(v)
    assert np.array_equal(got, code.astype(np.uint8))


def _f32_probe_values():
    rng = np.random.default_rng(2)
    bits = rng.integers(0, 2 ** 31, 400000, dtype=np.int64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    special = np.array([0.0, 1e-45, 1e-40, 5.96e-8, 2.98e-8, 6.1e-5, 65504.0, 65519.99,
                        65520.0, 65536.0, 1e5, 3.0e38, 3.4e38], np.float32)
    # exact bf16 ties: upper 16 bits plus half an ulp
    ties = (rng.integers(0, 2 ** 15, 20000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    allv = np.concatenate([v, special, ties, v * 1e-3])
    return np.concatenate([allv, -allv]).astype(np.float32)


def test_bf16_encoder_vs_torch(oracle):
    v = _f32_probe_values()
    got = oracle.enc_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_encoder_vs_torch(oracle):
    v = _f32_probe_values()
    got = oracle.enc_f16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_decoders_vs_torch(oracle):
    b = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    for mine, ref in ((oracle.bf16_value(b), R.bf16_to_f64(b)), (oracle.f16_value(b), R.f16_to_f64(b))):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(mine), nan)
        assert np.array_equal(mine[~nan], ref[~nan])


def test_softplus_vs_torch(oracle):
    v = np.concatenate([np.linspace(-30, 30, 10001), [-1e4, -745.0, 19.999, 20.0, 20.001, 50.0]])
    got = oracle.softplus(v)
    ref = R.softplus_torch(v)
    assert np.max(np.abs(got - ref) / (1e-300 + np.abs(ref))) < 4e-16
    assert oracle.softplus(np.array([-1e4]))[0] == 0.0


# --------------------------------------------------------------------------
# init
# --------------------------------------------------------------------------

@pytest.mark.parametrize("state_dtype", ["f32", "bf16", "f16", "fp8"])
@pytest.mark.parametrize("broadcast", [False, True])
def test_init_state_encodes_and_clears(oracle, state_dtype, broadcast):
    spec = synth.CacheSpec(num_slots=6, nheads=4, ngroups=2, headdim=8, dstate=16, ring_len=8,
                           state_dtype=state_dtype, slot_pad=32)
    cache = synth.make_cache(spec, 3)
    before = cache.copy()
    rng = np.random.default_rng(4)
    n = 4
    states = (rng.standard_normal((n, 4, 8, 16)) * 0.3).astype(np.float32)
    states[0, 1, 2, :] = 0.0  # an all-zero row: fp8 scale must be 1
    ids = np.array([2, 0, 5, 7], np.int32)  # 0 and 7 are ignored
    stride = 0 if broadcast else 4 * 8 * 16
    oracle.init_state(cache, states, ids, states_stride=stride)
    for j, slot in enumerate(ids):
        if slot <= 0 or slot >= spec.num_slots:
            continue
        src = states[0] if broadcast else states[j]
        raw = cache.state_logical(slot)
        if state_dtype == "f32":
            assert np.array_equal(raw, src)
        elif state_dtype == "bf16":
            assert np.array_equal(raw, torch.from_numpy(src).to(torch.bfloat16).view(torch.int16)
                                  .numpy().view(np.uint16))
        elif state_dtype == "f16":
            assert np.array_equal(raw, torch.from_numpy(src).to(torch.float16).view(torch.int16)
                                  .numpy().view(np.uint16))
        else:
            t = torch.from_numpy(src)
            m = t.abs().amax(dim=-1)
            scale = m / torch.tensor(448.0, dtype=torch.float32)
            scale = torch.where(scale > 0, scale, torch.ones_like(scale))
            assert np.array_equal(cache.scale_view(slot), scale.numpy())
            q = (t / scale[..., None]).clamp(-448, 448)
            codes = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            ok = (raw == codes) | (((raw & 0x7F) == 0) & ((codes & 0x7F) == 0))
            assert ok.all()
        assert not cache.x_view(slot).any() and not cache.B_view(slot).any()
        assert not cache.dt_view(slot).any() and cache.ring_start[slot] == 0
    # untouched: slots not listed, and every pad byte
    for slot in (0, 1, 3, 4):
        assert np.array_equal(cache.state[slot], before.state[slot])
        assert np.array_equal(cache.x_cache[slot], before.x_cache[slot])
        assert cache.ring_start[slot] == before.ring_start[slot]
    for name in ("state", "scale", "x_cache", "B_cache", "dt_cache"):
        a = getattr(cache, name)
        packed = {"state": spec.state_bytes(), "scale": spec.scale_bytes(), "x_cache": spec.x_bytes(),
                  "B_cache": spec.B_bytes(), "dt_cache": spec.dt_bytes()}[name]
        assert (a[:, packed:] == synth.CANARY).all(), name
