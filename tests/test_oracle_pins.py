"""Pins of the CPU oracle against what the pages and the mathematics fix.

The oracle computes the replay step as the plain sequential recurrence
h <- exp(A dt') h + dt' x B^T, y = h.C + D x (FlashInfer checkpointing-SSU
page, Description; vLLM replayssm_cutedsl page, selective_state_update_
replayssm).  These tests check it against independent routes to the same
numbers: the closed-form replay sum, arbitrary-precision brute force on tiny
shapes, flush invariants, the dt' -> 0 and A = 0 special cases, the causal
linear-attention form, ring rotation invariance and the textbook one-token
Mamba-2 update.  No GPU is used.
"""
import itertools

import mpmath
import numpy as np
import pytest
import torch

import synth
from tests import oracle_refs as R

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rel_err(a, b):
    return float(np.max(np.abs(a - b) / (1.0 + np.abs(b)))) if a.size else 0.0


def _small_case(state_dtype="f64", seed=0, H=4, G=2, P=8, N=16, L=8, T=3, batch=3,
                pnat_max=5, varlen=False, num_slots=6):
    spec = synth.CacheSpec(num_slots=num_slots, nheads=H, ngroups=G, headdim=P, dstate=N,
                           ring_len=L, state_dtype=state_dtype)
    cache = synth.make_cache(spec, seed)
    step = synth.make_step(spec, batch, T, seed + 1, pnat_max, varlen=varlen)
    return spec, cache, step


# --------------------------------------------------------------------------
# closed form
# --------------------------------------------------------------------------

@pytest.mark.parametrize("state_dtype", ["f64", "f32", "bf16", "f16", "fp8"])
@pytest.mark.parametrize("varlen", [False, True])
def test_closed_form_matches_sequential(oracle, state_dtype, varlen):
    spec, cache, step = _small_case(state_dtype, seed=3, varlen=varlen)
    before = cache.copy()
    out, status = oracle.replay_step(cache, step)
    assert status == 0
    for b in range(step.batch):
        for h in range(spec.nheads):
            seq = R.sequence(before, step, b, h)
            h0 = R.state_f64(before, seq["slot"])[h]
            ref = R.closed_form_outputs(h0, float(step.A[h]), float(step.D[h]), seq)
            got = out[seq["bos"]: seq["bos"] + seq["Tb"], h]
            assert _rel_err(got, ref) < 1e-12, (b, h)


def test_closed_form_at_full_head_shape(oracle):
    """P=64, N=128, L=16, T=8 with pnat up to 8: the production head shape."""
    spec, cache, step = _small_case("f32", seed=11, H=2, G=1, P=64, N=128, L=16, T=8,
                                    batch=2, pnat_max=8, num_slots=3)
    before = cache.copy()
    out, status = oracle.replay_step(cache, step)
    assert status == 0
    for b in range(step.batch):
        for h in range(spec.nheads):
            seq = R.sequence(before, step, b, h)
            h0 = R.state_f64(before, seq["slot"])[h]
            ref = R.closed_form_outputs(h0, float(step.A[h]), float(step.D[h]), seq)
            assert _rel_err(out[seq["bos"]: seq["bos"] + seq["Tb"], h], ref) < 1e-12


# --------------------------------------------------------------------------
# arbitrary-precision brute force on tiny shapes
# --------------------------------------------------------------------------

def _mp_replay(h0, A, D, seq, dps=50):
    """Explicit per-token state list in 50-digit arithmetic."""
    with mpmath.workdps(dps):
        P, N = h0.shape
        h = [[mpmath.mpf(float(h0[p, n])) for n in range(N)] for p in range(P)]
        A = mpmath.mpf(float(A))
        ys = []
        S = len(seq["dtp"])
        for s_ in range(S):
            d = mpmath.mpf(float(seq["dtp"][s_])) if s_ < seq["pnat"] else None
            if d is None:  # new token: softplus in arbitrary precision
                i = s_ - seq["pnat"]
                d = mpmath.log1p(mpmath.exp(mpmath.mpf(float(seq["_v"][i]))))
            dec = mpmath.exp(A * d)
            x = [mpmath.mpf(float(v)) for v in seq["x"][s_]]
            B = [mpmath.mpf(float(v)) for v in seq["B"][s_]]
            h = [[dec * h[p][n] + d * x[p] * B[n] for n in range(N)] for p in range(P)]
            if s_ >= seq["pnat"]:
                i = s_ - seq["pnat"]
                C = [mpmath.mpf(float(v)) for v in seq["C"][i]]
                ys.append([mpmath.fsum(h[p][n] * C[n] for n in range(N)) +
                           mpmath.mpf(float(D)) * x[p] for p in range(P)])
        return np.array([[float(v) for v in row] for row in ys])


@pytest.mark.parametrize("P,N,L,T", [(1, 1, 2, 1), (2, 3, 4, 3), (3, 2, 4, 2), (3, 3, 3, 3),
                                     (2, 1, 4, 1)])
def test_bruteforce_mpmath_tiny(oracle, P, N, L, T):
    spec, cache, step = _small_case("f64", seed=5 + P * 7 + N, H=2, G=1, P=P, N=N, L=L, T=T,
                                    batch=2, pnat_max=L - T, num_slots=4)
    before = cache.copy()
    out, status = oracle.replay_step(cache, step)
    assert status == 0
    for b in range(step.batch):
        for h in range(spec.nheads):
            seq = R.sequence(before, step, b, h)
            toks = np.arange(seq["bos"], seq["bos"] + seq["Tb"])
            seq["_v"] = step.dt[toks, h].astype(np.float64) + float(step.dt_bias[h])
            h0 = R.state_f64(before, seq["slot"])[h]
            ref = _mp_replay(h0, step.A[h], step.D[h], seq)
            assert _rel_err(out[toks, h], ref) < 1e-13


# --------------------------------------------------------------------------
# flush invariants (fp64 state: exact)
# --------------------------------------------------------------------------

def test_flush_equals_sequential_state(oracle):
    """replay_step(p, T) then flush(k) leaves the checkpoint equal to the
    state after running the first k tokens sequentially (closed form)."""
    spec, cache, step = _small_case("f64", seed=21, pnat_max=5, T=3)
    before = cache.copy()
    oracle.replay_step(cache, step)
    after_step = cache.copy()
    k = np.array([min(int(p) + 2, spec.ring_len) for p in step.pnat], np.int32)
    st = oracle.flush(cache, step.slot_idx, k, step.A)
    assert st == 0
    L = spec.ring_len
    for j, slot in enumerate(step.slot_idx):
        r = int(after_step.ring_start[slot])
        pos = [(r + s_) % L for s_ in range(k[j])]
        for h in range(spec.nheads):
            g = h // (spec.nheads // spec.ngroups)
            h0 = R.state_f64(before, slot)[h]
            ref = R.closed_form_state(h0, float(step.A[h]),
                                      after_step.dt_view(slot)[h][pos].astype(np.float64),
                                      R.bf16_to_f64(after_step.x_view(slot)[h][pos]),
                                      R.bf16_to_f64(after_step.B_view(slot)[g][pos]))
            got = R.state_f64(cache, slot)[h]
            assert _rel_err(got, ref) < 1e-12
        assert cache.ring_start[slot] == (r + k[j]) % L


def test_flush_then_step_invariance(oracle):
    """Outputs of step(p, T) equal those of flush(k <= p) then step(p - k, T)
    (fp64 state: the same operations in the same order, so bit-identical)."""
    spec, cache, step = _small_case("f64", seed=31, pnat_max=5, T=3, batch=4, num_slots=8)
    ref_out, _ = oracle.replay_step(cache.copy(), step)
    k = np.array([int(p) // 2 + (int(p) % 2) for p in step.pnat], np.int32)  # 0..p
    c2 = cache.copy()
    assert oracle.flush(c2, step.slot_idx, k, step.A) == 0
    step2 = synth.StepInputs(**{**step.__dict__, "pnat": (step.pnat - k).astype(np.int32)})
    out2, st = oracle.replay_step(c2, step2)
    assert st == 0
    assert np.array_equal(out2, ref_out)


def test_z_gate_closed_form(oracle):
    """Gated readout: the closed form times z sigmoid(z), z through torch's
    bf16 decode and torch's sigmoid (independent of the oracle's C)."""
    spec = synth.CacheSpec(num_slots=6, nheads=4, ngroups=2, headdim=8, dstate=16, ring_len=8,
                           state_dtype="f64")
    cache = synth.make_cache(spec, 13)
    step = synth.make_step(spec, 3, 3, 14, 5, with_z=True)
    out, st = oracle.replay_step(cache.copy(), step)
    assert st == 0
    zv = R.bf16_to_f64(step.z)
    gate = zv * torch.sigmoid(torch.from_numpy(zv)).numpy()
    for b in range(step.batch):
        h0 = R.state_f64(cache, int(step.slot_idx[b]))
        for h in range(spec.nheads):
            seq = R.sequence(cache, step, b, h)
            want = R.closed_form_outputs(h0[h], float(step.A[h]), float(step.D[h]), seq)
            rows = slice(seq["bos"], seq["bos"] + seq["Tb"])
            assert _rel_err(out[rows, h], want * gate[rows, h]) <= 1e-12
    step.z[:] = 0  # silu(0) = 0: every output is exactly zero
    out0, _ = oracle.replay_step(cache.copy(), step)
    assert np.all(out0 == 0.0)


def test_dt_softplus_off_closed_form(oracle):
    """dt_softplus = False: dt' = dt + dt_bias, in the readout and in the
    appended dt ring."""
    spec = synth.CacheSpec(num_slots=6, nheads=4, ngroups=2, headdim=8, dstate=16, ring_len=8,
                           state_dtype="f64")
    cache = synth.make_cache(spec, 23)
    step = synth.make_step(spec, 3, 3, 24, 5, dt_softplus=False)
    c2 = cache.copy()
    out, st = oracle.replay_step(c2, step)
    assert st == 0
    L = spec.ring_len
    for b in range(step.batch):
        slot = int(step.slot_idx[b])
        h0 = R.state_f64(cache, slot)
        for h in range(spec.nheads):
            seq = R.sequence(cache, step, b, h)
            want = R.closed_form_outputs(h0[h], float(step.A[h]), float(step.D[h]), seq)
            rows = slice(seq["bos"], seq["bos"] + seq["Tb"])
            assert _rel_err(out[rows, h], want) <= 1e-12
            for i in range(seq["Tb"]):
                pos = (int(cache.ring_start[slot]) + seq["pnat"] + i) % L
                want_dt = np.float32(step.dt[seq["bos"] + i, h]) + np.float32(step.dt_bias[h])
                assert c2.dt_view(slot)[h, pos] == want_dt
    # and it differs from the softplus run
    step.dt_softplus = True
    out_sp, _ = oracle.replay_step(cache.copy(), step)
    assert not np.allclose(out_sp, out)


def test_fused_flush_in_step_f64(oracle):
    """The fused call (fold k <= pnat live tokens, then step) reads out exactly
    what the plain step reads out (fp64 state), leaves the checkpoint at the
    closed-form state after the k folded tokens, and advances ring_start by k."""
    spec, cache, step = _small_case("f64", seed=37, pnat_max=5, T=3, batch=4, num_slots=8)
    rng = np.random.default_rng(3)
    k = np.array([rng.integers(0, int(p) + 1) for p in step.pnat], np.int32)
    k[int(np.argmax(step.pnat))] = int(np.max(step.pnat))  # one entry folds its whole prefix
    ref_out, _ = oracle.replay_step(cache.copy(), step)
    c2 = cache.copy()
    out2, st = oracle.replay_step(c2, step, num_fold=k)
    assert st == 0
    assert np.array_equal(out2, ref_out)
    L = spec.ring_len
    for b in range(step.batch):
        slot, kb = int(step.slot_idx[b]), int(k[b])
        assert int(c2.ring_start[slot]) == (int(cache.ring_start[slot]) + kb) % L
        h0 = R.state_f64(cache, slot)
        got = R.state_f64(c2, slot)
        for h in range(spec.nheads):
            seq = R.sequence(cache, step, b, h)
            want = R.closed_form_state(h0[h], float(step.A[h]), seq["dtp"][:kb], seq["x"][:kb],
                                       seq["B"][:kb])
            assert _rel_err(got[h], want) <= 1e-12


def test_fused_invalid_fold_is_skipped(oracle):
    spec, cache, step = _small_case("f32", seed=41, pnat_max=4, T=2, batch=4, num_slots=8)
    step.pnat[:] = [2, 3, 1, 0]
    k = np.array([1, 4, -1, 0], np.int32)  # entries 1 (k > pnat) and 2 (k < 0) are invalid
    before = cache.copy()
    out, st = oracle.replay_step(cache, step, num_fold=k)
    assert st == 2
    T = step.T
    assert np.all(out[1 * T:3 * T] == 0.0)
    for b in (1, 2):
        slot = int(step.slot_idx[b])
        assert np.array_equal(cache.state[slot], before.state[slot])
        assert np.array_equal(cache.x_cache[slot], before.x_cache[slot])
        assert int(cache.ring_start[slot]) == int(before.ring_start[slot])
    s0 = int(step.slot_idx[0])
    assert int(cache.ring_start[s0]) == (int(before.ring_start[s0]) + 1) % spec.ring_len
    assert not np.array_equal(cache.state[s0], before.state[s0])


# --------------------------------------------------------------------------
# special cases
# --------------------------------------------------------------------------

def _zero_dt(cache, step):
    for s_ in range(cache.spec.num_slots):
        cache.dt_view(s_)[:] = 0.0
    step.dt[:] = -1.0e4  # softplus(-1e4 + bias) is exactly 0 in fp64
    return cache, step


@pytest.mark.parametrize("state_dtype", ["f32", "bf16", "f16", "fp8"])
def test_dt_zero_identity(oracle, state_dtype):
    """dt' = 0 everywhere: y = C.h0 + D x, and a flush leaves the checkpoint
    unchanged (fp8: identical codes and scales when each row's largest code is
    448, within one ulp of the scale)."""
    spec, cache, step = _small_case(state_dtype, seed=41, pnat_max=5, T=3)
    cache, step = _zero_dt(cache, step)
    if state_dtype == "fp8":
        for s_ in range(spec.num_slots):
            v = cache.state_logical(s_)
            v[:, :, 0] = 0x7E  # +448 in every row
            cache.set_state_logical(s_, v)
    before = cache.copy()
    out, st = oracle.replay_step(cache, step)
    assert st == 0
    for b in range(step.batch):
        slot = int(step.slot_idx[b])
        for h in range(spec.nheads):
            g = h // (spec.nheads // spec.ngroups)
            h0 = R.state_f64(before, slot)[h]
            toks = np.arange(b * step.T, (b + 1) * step.T)
            ref = (R.bf16_to_f64(step.C[toks, g]) @ h0.T +
                   float(step.D[h]) * R.bf16_to_f64(step.x[toks, h]))
            assert _rel_err(out[toks, h], ref) < 1e-13
    k = np.full(step.batch, 3, np.int32)
    mid = cache.copy()
    assert oracle.flush(cache, step.slot_idx, k, step.A) == 0
    for slot in step.slot_idx:
        assert np.array_equal(cache.state_view(slot), mid.state_view(slot))
        if state_dtype == "fp8":
            a = cache.scale_view(slot).view(np.int32).astype(np.int64)
            b_ = mid.scale_view(slot).view(np.int32).astype(np.int64)
            assert np.max(np.abs(a - b_)) <= 1


def test_A_zero_flush_is_plain_sum(oracle):
    """A = 0: the fold is h0 + sum_s dt'_s x_s B_s^T (an einsum)."""
    spec, cache, step = _small_case("f64", seed=51, pnat_max=5, T=3)
    step.A[:] = 0.0
    before = cache.copy()
    oracle.replay_step(cache, step)
    after = cache.copy()
    k = np.full(step.batch, 5, np.int32)
    oracle.flush(cache, step.slot_idx, k, step.A)
    L = spec.ring_len
    for slot in step.slot_idx:
        r = int(after.ring_start[slot])
        pos = [(r + s_) % L for s_ in range(5)]
        for h in range(spec.nheads):
            g = h // (spec.nheads // spec.ngroups)
            ref = R.state_f64(before, slot)[h] + np.einsum(
                "s,sp,sn->pn", after.dt_view(slot)[h][pos].astype(np.float64),
                R.bf16_to_f64(after.x_view(slot)[h][pos]),
                R.bf16_to_f64(after.B_view(slot)[g][pos]))
            assert _rel_err(R.state_f64(cache, slot)[h], ref) < 1e-13


def test_A_zero_h0_zero_is_causal_linear_attention(oracle):
    """A = 0, h0 = 0: Y = (mask o (C B^T) diag(dt')) X + D x_new."""
    spec, cache, step = _small_case("f64", seed=61, pnat_max=5, T=3)
    step.A[:] = 0.0
    for s_ in range(spec.num_slots):
        cache.state_view(s_)[:] = 0.0  # zero in any layout
    before = cache.copy()
    out, _ = oracle.replay_step(cache, step)
    for b in range(step.batch):
        for h in range(spec.nheads):
            seq = R.sequence(before, step, b, h)
            p, Tb = seq["pnat"], seq["Tb"]
            S = p + Tb
            M = np.zeros((Tb, S))
            for i in range(Tb):
                M[i, : p + i + 1] = 1.0
            Y = (M * (seq["C"] @ seq["B"].T) * seq["dtp"][None, :]) @ seq["x"]
            Y = Y + float(step.D[h]) * seq["xnew"]
            assert _rel_err(out[seq["bos"]: seq["bos"] + Tb, h], Y) < 1e-13


def test_ring_rotation_invariance(oracle):
    """The same logical sequence stored at ring_start r and at (r + d) mod L
    gives bit-identical outputs, and the appends land rotated by d."""
    spec, cache, step = _small_case("f32", seed=71, pnat_max=5, T=3)
    L = spec.ring_len
    out1, _ = oracle.replay_step(cache.copy(), step)
    for d in (1, 3, L - 1):
        c2 = cache.copy()
        for slot in range(spec.num_slots):
            for view in (c2.x_view, c2.B_view, c2.dt_view):
                v = view(slot)
                v[:] = np.roll(v.copy(), d, axis=1)
            c2.ring_start[slot] = (cache.ring_start[slot] + d) % L
        ref_cache = cache.copy()
        oracle.replay_step(ref_cache, step)
        out2, _ = oracle.replay_step(c2, step)
        assert np.array_equal(out1, out2)
        for slot in step.slot_idx:
            assert np.array_equal(np.roll(ref_cache.x_view(slot), d, axis=1), c2.x_view(slot))
            assert np.array_equal(np.roll(ref_cache.dt_view(slot), d, axis=1), c2.dt_view(slot))


def test_single_token_textbook_update(oracle):
    """T = 1, pnat = 0 is one Mamba-2 selective state update:
    dA = exp(dt' A), h' = dA h + dt' x B^T, y = h' C + D x; and a flush of that
    one token stores exactly h'."""
    spec, cache, step = _small_case("f64", seed=81, T=1, pnat_max=0)
    before = cache.copy()
    out, _ = oracle.replay_step(cache, step)
    oracle.flush(cache, step.slot_idx, np.ones(step.batch, np.int32), step.A)
    for b in range(step.batch):
        slot = int(step.slot_idx[b])
        for h in range(spec.nheads):
            g = h // (spec.nheads // spec.ngroups)
            dtp = R.softplus_torch(np.array([step.dt[b, h] + np.float64(step.dt_bias[h])]))[0]
            x = R.bf16_to_f64(step.x[b, h])
            Bv = R.bf16_to_f64(step.B[b, g])
            Cv = R.bf16_to_f64(step.C[b, g])
            hn = np.exp(dtp * float(step.A[h])) * R.state_f64(before, slot)[h] + dtp * np.outer(x, Bv)
            assert _rel_err(out[b, h], hn @ Cv + float(step.D[h]) * x) < 1e-13
            # the flush reads dt' back from the f32 dt ring
            d32 = float(np.float32(dtp))
            hf = np.exp(d32 * float(step.A[h])) * R.state_f64(before, slot)[h] + d32 * np.outer(x, Bv)
            assert _rel_err(R.state_f64(cache, slot)[h], hf) < 1e-14


def test_varlen_equals_per_sequence(oracle):
    """A packed varlen call equals separate calls with T = T_b per entry."""
    spec, cache, step = _small_case("f32", seed=91, varlen=True, T=3, pnat_max=5, batch=4,
                                    num_slots=8)
    out, st = oracle.replay_step(cache.copy(), step)
    assert st == 0
    for b in range(step.batch):
        lo, hi = int(step.cu_seqlens[b]), int(step.cu_seqlens[b + 1])
        one = synth.StepInputs(1, hi - lo, step.slot_idx[b:b + 1], step.pnat[b:b + 1], None,
                               step.x[lo:hi], step.B[lo:hi], step.C[lo:hi], step.dt[lo:hi],
                               step.A, step.D, step.dt_bias)
        o1, _ = oracle.replay_step(cache.copy(), one)
        assert np.array_equal(o1, out[lo:hi])


def test_padding_and_invalid_entries(oracle):
    spec, cache, step = _small_case("f32", seed=101, T=3, pnat_max=5, batch=4, num_slots=8)
    step.slot_idx[0] = 0  # padding
    step.slot_idx[1] = spec.num_slots  # out of range: padding
    step.pnat[2] = spec.ring_len - 2  # pnat + T > L: invalid
    before = cache.copy()
    out, st = oracle.replay_step(cache, step)
    assert st == 1
    assert np.all(out[0:9] == 0.0)
    for slot in (0, int(step.slot_idx[2])):
        for a, b_ in ((cache.x_view(slot), before.x_view(slot)),
                      (cache.dt_view(slot), before.dt_view(slot))):
            assert np.array_equal(a, b_)
    assert np.all(np.isfinite(out[9:]))
    k = np.array([2, 2, spec.ring_len + 1, -1], np.int32)
    st = oracle.flush(cache, step.slot_idx, k, step.A)
    assert st == 2


@pytest.mark.parametrize("bad", [-1, 16, 40])
def test_bad_ring_start_is_skipped(oracle, bad):
    """A slot whose ring_start lies outside [0, L) has no live or append
    position under the ring contract (FlashInfer PR, Description item 2):
    the step writes zero output rows for its entry, touches none of its
    cache and raises status bit 8; the flush leaves it alone and raises the
    same bit; the other entries are computed as if it were absent."""
    spec, cache, step = _small_case("f32", seed=103, T=2, pnat_max=3, batch=3, num_slots=6)
    slot = int(step.slot_idx[1])
    cache.ring_start[slot] = bad
    before = cache.copy()
    out, st = oracle.replay_step(cache, step)
    assert st == 8
    assert np.all(out[2:4] == 0.0)
    for f in ("x_cache", "B_cache", "dt_cache", "state"):
        assert np.array_equal(getattr(cache, f)[slot], getattr(before, f)[slot]), f
    # the other entries: as in a call without the bad one
    keep = [0, 2]
    sub = synth.StepInputs(2, step.T, step.slot_idx[keep], step.pnat[keep], None,
                           np.concatenate([step.x[0:2], step.x[4:6]]), np.concatenate([step.B[0:2], step.B[4:6]]),
                           np.concatenate([step.C[0:2], step.C[4:6]]), np.concatenate([step.dt[0:2], step.dt[4:6]]),
                           step.A, step.D, step.dt_bias)
    o2, st2 = oracle.replay_step(before.copy(), sub)
    assert st2 == 0
    assert np.array_equal(np.concatenate([out[0:2], out[4:6]]), o2)
    k = np.array([1, 2, 1], np.int32)
    c2 = before.copy()
    assert oracle.flush(c2, step.slot_idx, k, step.A) == 8
    assert c2.ring_start[slot] == bad
    assert np.array_equal(c2.state[slot], before.state[slot])
    for b in (0, 2):
        sl = int(step.slot_idx[b])
        assert c2.ring_start[sl] == (before.ring_start[sl] + k[b]) % spec.ring_len


# --------------------------------------------------------------------------
# ring contract fixture (positions fixed by the page's formula)
# --------------------------------------------------------------------------

def _load_ring_fixture():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "ring_positions.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        r, p, T, L, live, app = line.split("|")
        rows.append((int(r), int(p), int(T), int(L),
                     [int(v) for v in live.split()] if live.strip() else [],
                     [int(v) for v in app.split()]))
    return rows


@pytest.mark.parametrize("row", _load_ring_fixture())
def test_ring_positions_fixture(oracle, row):
    """Appends land where the ring contract says, and only there."""
    r, p, T, L, live, app = row
    spec = synth.CacheSpec(num_slots=2, nheads=1, ngroups=1, headdim=2, dstate=2, ring_len=L,
                           state_dtype="f64")
    cache = synth.make_cache(spec, 7)
    cache.ring_start[1] = r
    step = synth.make_step(spec, 1, T, 8, 0, slots=np.array([1], np.int32), pnat_fixed=p)
    before = cache.copy()
    oracle.replay_step(cache, step)
    changed = [j for j in range(L)
               if not np.array_equal(cache.x_view(1)[0, j], before.x_view(1)[0, j])]
    assert sorted(changed) == sorted(app)
    for i, pos in enumerate(app):
        assert np.array_equal(cache.x_view(1)[0, pos], step.x[i, 0])
        assert np.array_equal(cache.B_view(1)[0, pos], step.B[i, 0])
    # the live entries are the ones the output depends on: perturb each one
    out0, _ = oracle.replay_step(before.copy(), step)
    for j in range(L):
        c2 = before.copy()
        c2.dt_view(1)[0, j] += 0.25
        o2, _ = oracle.replay_step(c2, step)
        assert (not np.array_equal(o2, out0)) == (j in live), j
