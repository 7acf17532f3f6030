"""Pins of the oracle's NVFP4 read checkpoint (CPU only).

vLLM PR "Add separate CuTeDSL ReplaySSM checkpoints" (Overview, Claims):
FP8/NVFP4 read checkpoints with nearest encoding beside the FP16 recurrence
checkpoint.  vLLM API page "replayssm_cutedsl", initialize_replayssm_state,
NVFP4 branch: the largest |value| of each group of heads, then the maximum
of those over the groups divided by 6 * 448 gives ONE second-level scale per
slot (1 where it is not positive; a stride-0 batch of states broadcasts the
first state's).  Reading (also in the oracle's header): e2m1 elements, an e4m3
scale per 16 values along dstate; a fold re-encodes the whole slot the same
way from its folded fp32 state.

Pinned against: the page's own torch lines for the second-level scale
(page_global_scale below, run on torch CPU), the E2M1 value table of the OCP
Microscaling Formats specification (v1.0, FP4 E2M1), brute-force nearest
searches for both levels written here in numpy, exact round trips of
representable slots, an independent numpy statement of the byte layout, the
replay reduced to the fp64-state oracle on the decoded values, and a
separate-checkpoint flush against the numpy closed form.
"""
import numpy as np
import pytest
import torch

import synth
from tests import oracle_refs as R

# OCP MX v1.0, FP4 E2M1: codes 0..7 (sign bit 3 clear)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E4M3_VALUES = R.e4m3_to_f64(np.arange(127, dtype=np.uint8))  # codes 0x00..0x7E


def test_e2m1_values(oracle):
    codes = np.arange(16, dtype=np.uint8)
    want = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])
    got = oracle.e2m1_value(codes)
    assert np.array_equal(got, want)
    assert np.signbit(got[8])  # code 8 is negative zero


def _nearest(table, a):
    """Index of the nearest table entry to a >= 0 (ties to the even index);
    past the last entry the last one (saturation)."""
    d = np.abs(np.asarray(table)[None, :] - np.asarray(a, np.float64)[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(len(table))[None, :] % 2 == 0)
    idx = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return idx


def e2m1_encode_ref(q):
    q = np.asarray(q, np.float64)
    code = _nearest(E2M1_TABLE, np.abs(q).ravel()).astype(np.uint8).reshape(q.shape)
    return code | np.where(np.signbit(q), 8, 0).astype(np.uint8)


def test_e2m1_encoder_is_nearest(oracle):
    rng = np.random.default_rng(1)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    v = np.concatenate([rng.uniform(-8, 8, 4000), mids, [-m for m in mids], E2M1_TABLE,
                        [6.0001, 7.0, 100.0, -100.0, 1e-30, -1e-30, 0.0, -0.0]])
    got = oracle.enc_e2m1(v)
    assert np.array_equal(got, e2m1_encode_ref(v))
    # ties go to the even code: 0.25 -> 0, 0.75 -> 1.0, 2.5 -> 2, 5 -> 4
    assert list(oracle.enc_e2m1(np.array([0.25, 0.75, 2.5, 5.0]))) == [0, 2, 4, 6]
    assert oracle.enc_e2m1(np.array([-0.0]))[0] == 8 and oracle.enc_e2m1(np.array([-0.1]))[0] == 8


def page_global_scale(states, groups):
    """The second-level scale of each entry of FP32 prefill states
    [batch, heads, 64, 128], as the NVFP4 branch of initialize_replayssm_state
    on the vLLM API page computes it (torch on the CPU): the largest |value| of
    every group of heads, their maximum over the groups divided by 6 * 448,
    and 1 where that is not positive."""
    st = torch.as_tensor(np.ascontiguousarray(states, np.float32))
    heads = st.shape[1]
    group_max = st.abs().reshape(-1, groups, (heads // groups) * 64 * 128).amax(dim=-1)
    global_scale = group_max.amax(dim=-1) / (6.0 * 448.0)
    global_scale = torch.where(global_scale > 0, global_scale, 1.0)
    return global_scale.numpy()


def nvfp4_encode_ref(hv, g):
    """NVFP4 encoding of one head [P, N] of fp32 values with second-level
    scale g, by the definition in numpy float32 with brute-force nearest
    searches: (codes [P, N], block scale codes [P, N / 16])."""
    hv = np.asarray(hv, np.float32)
    g = np.float32(g)
    ds = np.float32(6.0) * g
    P, N = hv.shape
    blocks = hv.reshape(P, N // 16, 16)
    a = np.max(np.abs(blocks), axis=2)
    t = (a / ds).astype(np.float32)
    sf = _nearest(E4M3_VALUES, np.minimum(t.astype(np.float64), 448.0).ravel()).reshape(t.shape).astype(np.uint8)
    es = (E4M3_VALUES[sf].astype(np.float32) * g).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(es[:, :, None] > 0, blocks / es[:, :, None], np.float32(0.0) * blocks).astype(np.float32)
    return e2m1_encode_ref(q).reshape(P, N), sf


def decode_ref(codes, sf, g):
    vals = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE])[codes]
    P, N = codes.shape
    return (vals.reshape(P, N // 16, 16) * E4M3_VALUES[sf][:, :, None] * np.float64(g)).reshape(P, N)


def _spec(layout="", separate=False, nheads=2, ngroups=1):
    return synth.CacheSpec(num_slots=4, nheads=nheads, ngroups=ngroups, state_dtype="nvfp4", state_layout=layout,
                           separate=separate)


def _tiled_code_pos(p, n):
    rb, m, q, t = p // 16, p % 16, n // 32, n % 32
    lane = 16 * q + m
    return rb * 1024 + lane * 16 + t // 2, t % 2


def _tiled_scale_pos(p, n):
    rb, m, q, t = p // 16, p % 16, n // 32, n % 32
    return (16 * q + m) * 8 + rb * 2 + t // 16


def _check_head_bytes(cache, slot, h, codes, sf, layout):
    raw = cache.state_view(slot)[h]
    sraw = cache.scale_view(slot)[h]
    for p in range(64):
        for n in range(128):
            if layout == "tiled":
                byte, hi = _tiled_code_pos(p, n)
                s_at = _tiled_scale_pos(p, n)
            else:
                byte, hi = (p * 128 + n) // 2, (p * 128 + n) % 2
                s_at = p * 8 + n // 16
            code = (raw[byte] >> 4) if hi else (raw[byte] & 15)
            assert code == codes[p, n], (p, n, code, codes[p, n])
            assert sraw[s_at] == sf[p, n // 16]


@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
def test_nvfp4_encode_matches_reference(oracle, layout):
    """A slot of four heads in two groups: the second-level scale is the
    page's, shared by every head; head 3 sits far below the slot maximum, so
    its block scales are those of the slot's scale, not of its own maximum."""
    spec = _spec(layout, nheads=4, ngroups=2)
    cache = synth.make_cache(spec, 5)
    rng = np.random.default_rng(2)
    hv = (rng.standard_normal((4, 64, 128)) * rng.uniform(0.01, 3.0, (4, 64, 1))).astype(np.float32)
    hv[0, 3, 16:32] = 0.0           # a zero block
    hv[1, 5, :] *= np.float32(1e-6)  # blocks far below the slot maximum (tiny or zero block scales)
    hv[3] *= np.float32(1e-3)        # a whole head far below the slot maximum
    oracle.encode_slot_nvfp4(cache, 2, hv)
    g = page_global_scale(hv[None], 2)[0]
    words = cache.gscale_view(2)
    assert words[0] == g
    assert np.array_equal(words[1:], np.max(np.abs(hv).reshape(4, -1), axis=1))
    dec = oracle.decode_state(cache, 2)
    for h in range(4):
        codes, sf = nvfp4_encode_ref(hv[h], g)
        _check_head_bytes(cache, 2, h, codes, sf, layout)
        assert np.array_equal(dec[h], decode_ref(codes, sf, g))
        # every element lies within half an e2m1 step (at most one unit of es) of
        # its value, or saturates at 6 es where a block scale rounded down (a
        # block far below the slot maximum has a subnormal e4m3 scale); a block
        # whose scale rounds to zero held values below 6 g 2^-10 (half the
        # smallest e4m3 value) and decodes to zero
        es = E4M3_VALUES[sf].astype(np.float64) * np.float64(g)
        es = np.where(sf == 0, 6.0 * np.float64(g) * 2.0 ** -10, es)[:, :, None]
        err = np.abs(dec[h] - hv[h]).reshape(64, 8, 16)
        sat = np.maximum(np.abs(hv[h]).reshape(64, 8, 16) - 6.0 * es, 0.0)
        assert np.all(err <= es + sat + 1e-30)
        # a normal block scale rounds the block maximum down by under 1/16, so
        # saturation stays within the half step there
        assert np.all(err[sf >= 8] <= es[sf >= 8] + 1e-30)
    # the small head's own maximum would give it other block scales
    own = page_global_scale(hv[3][None, None], 1)[0]
    assert not np.array_equal(nvfp4_encode_ref(hv[3], own)[1], nvfp4_encode_ref(hv[3], g)[1])
    assert np.any(nvfp4_encode_ref(hv[1], g)[1][5] == 0)  # the tiny blocks
    assert np.max(np.abs(dec)) == pytest.approx(np.max(np.abs(hv)), rel=0.07)


def test_nvfp4_representable_slots_round_trip(oracle):
    """A slot built from e2m1 codes, e4m3 block scales and a power-of-two
    second-level scale, with the slot maximum at 6 * 448 * g and every block
    maximum at 6 * its scale, encodes back to the same codes and scales."""
    spec = _spec("tiled")
    cache = synth.make_cache(spec, 7)
    rng = np.random.default_rng(3)
    g = np.float32(2.0 ** -9)
    hv = np.empty((2, 64, 128), np.float32)
    want = []
    for h in range(2):
        sf = rng.integers(0x20, 0x7E, (64, 8)).astype(np.uint8)  # normal e4m3 values 2^-3 .. 448
        if h == 1:
            sf[0, 0] = 0x7E  # 448: the slot maximum sits in head 1
        codes = rng.integers(0, 16, (64, 128)).astype(np.uint8)
        codes.reshape(64, 8, 16)[:, :, 0] = 7  # a +6 in every block
        hv[h] = decode_ref(codes, sf, g).astype(np.float32)
        assert np.array_equal(hv[h].astype(np.float64), decode_ref(codes, sf, g))  # exact in fp32
        want.append((codes, sf))
    oracle.encode_slot_nvfp4(cache, 1, hv)
    assert cache.gscale_view(1)[0] == g == page_global_scale(hv[None], 1)[0]
    dec = oracle.decode_state(cache, 1)
    assert np.array_equal(dec, hv.astype(np.float64))
    for h, (codes, sf) in enumerate(want):
        got_codes, got_sf = nvfp4_encode_ref(hv[h], g)
        assert np.array_equal(got_sf, sf)
        zero = (codes & 7) == 0  # negative zero codes decode to zero: compare values there
        assert np.array_equal(got_codes[~zero], codes[~zero])


def test_nvfp4_zero_slot_uses_unit_scale(oracle):
    spec = _spec("tiled")
    cache = synth.make_cache(spec, 8)
    oracle.encode_slot_nvfp4(cache, 3, np.zeros((2, 64, 128), np.float32))
    assert cache.gscale_view(3)[0] == 1.0 == page_global_scale(np.zeros((1, 2, 64, 128)), 1)[0]
    assert np.all(oracle.decode_state(cache, 3) == 0.0)


def test_nvfp4_replay_is_the_replay_of_the_decoded_state(oracle):
    """The step reads the NVFP4 checkpoint as its decoded values: the same
    step on an fp64 copy holding those values gives the same outputs."""
    spec = synth.CacheSpec(num_slots=6, nheads=4, ngroups=2, state_dtype="nvfp4")
    cache = synth.make_cache(spec, 21)
    step = synth.make_step(spec, 4, 3, 22, 6)
    out, st = oracle.replay_step(cache.copy(), step)
    assert st == 0
    s64 = synth.CacheSpec(**{**spec.__dict__, "state_dtype": "f64", "state_layout": "rowmajor"})
    c64 = synth.CacheArrays(s64, np.zeros((spec.num_slots, s64.strides()["state"]), np.uint8),
                            np.zeros((spec.num_slots, s64.strides()["scale"]), np.uint8),
                            cache.x_cache.copy(), cache.B_cache.copy(), cache.dt_cache.copy(),
                            cache.ring_start.copy())
    for sl in range(1, spec.num_slots):
        c64.set_state_logical(sl, oracle.decode_state(cache, sl))
    ref, st = oracle.replay_step(c64, step)
    assert st == 0
    assert np.max(np.abs(out - ref)) <= 1e-12 * (1 + np.max(np.abs(ref)))


def test_nvfp4_separate_flush_closed_form(oracle):
    """Separate flush into an NVFP4 read checkpoint: the read checkpoint is
    the reference NVFP4 encoding of fp32(closed-form state folded from the
    FP16 recurrence checkpoint), with the slot scale taken, as at init, over
    every head of the folded slot."""
    spec = synth.CacheSpec(num_slots=6, nheads=4, ngroups=2, state_dtype="nvfp4", separate=True)
    cache = synth.make_cache(spec, 31)
    step = synth.make_step(spec, 4, 3, 32, 5)
    c = cache.copy()
    oracle.replay_step(c, step)
    before = c.copy()
    k = np.array([min(int(p) + 2, spec.ring_len) for p in step.pnat], np.int32)
    assert oracle.flush(c, step.slot_idx, k, step.A, 1234) == 0
    agree = []
    for b in range(step.batch):
        slot = int(step.slot_idx[b])
        h0 = oracle.decode_recur(before, slot)
        dec = oracle.decode_state(c, slot)
        want = np.empty((spec.nheads, 64, 128), np.float32)
        for h in range(spec.nheads):
            seq = R.sequence(before, synth.StepInputs(**{**step.__dict__, "pnat": k}), b, h)
            want[h] = R.closed_form_state(h0[h], float(step.A[h]), seq["dtp"][: k[b]], seq["x"][: k[b]],
                                          seq["B"][: k[b]]).astype(np.float32)
        g = page_global_scale(want[None], spec.ngroups)[0]
        assert abs(c.gscale_view(slot)[0] - g) <= 2.0 ** -22 * g
        for h in range(spec.nheads):
            codes, sf = nvfp4_encode_ref(want[h], g)
            ref = decode_ref(codes, sf, g)
            agree.append(np.mean(np.abs(dec[h] - ref) <= 1e-6 * np.abs(ref) + 1e-30))
    assert min(agree) >= 0.999, min(agree)
    assert np.array_equal(c.ring_start[step.slot_idx], (before.ring_start[step.slot_idx] + k) % spec.ring_len)


@pytest.mark.parametrize("broadcast", [False, True])
def test_nvfp4_init_follows_the_page(oracle, broadcast):
    """Init from FP32 prefill states: the slot scale bit for bit as the page's
    torch lines compute it (two groups of two heads, one state all zero),
    codes and block scales as the reference encoding with that scale, the
    rings cleared; a stride-0 batch gives every slot the first state's scale."""
    spec = synth.CacheSpec(num_slots=6, nheads=4, ngroups=2, state_dtype="nvfp4", separate=True)
    cache = synth.make_cache(spec, 41)
    rng = np.random.default_rng(9)
    states = (rng.standard_normal((3, 4, 64, 128)) * rng.uniform(0.05, 0.5, (3, 4, 1, 1))).astype(np.float32)
    states[2] = 0.0
    slots = np.array([3, 1, 5], np.int32)
    if broadcast:
        oracle.init_state(cache, states[:1], slots, states_stride=0, seed=5)
        src = np.broadcast_to(states[:1], states.shape)
        want_g = np.repeat(page_global_scale(states[:1], 2), 3)
    else:
        oracle.init_state(cache, states, slots, seed=5)
        src = states
        want_g = page_global_scale(states, 2)
    assert want_g[-1] == 1.0 or broadcast
    for j, slot in enumerate(slots):
        assert cache.gscale_view(slot)[0] == want_g[j]
        dec = oracle.decode_state(cache, slot)
        for h in range(4):
            codes, sf = nvfp4_encode_ref(src[j, h], want_g[j])
            assert np.array_equal(dec[h], decode_ref(codes, sf, want_g[j]))
        assert np.all(cache.x_view(slot) == 0) and cache.ring_start[slot] == 0
