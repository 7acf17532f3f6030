"""Helpers shared by the GPU tests: run the library on synth inputs and compare
with the oracle.  Imported only by tests marked `gpu`."""
from __future__ import annotations

import numpy as np
import torch

import speculative_replay_state_amd as ssu
import synth
from synth import device as sd

DEV = "cuda:0"


def device_cache(spec: synth.CacheSpec, t: dict, with_status: bool = True) -> ssu.DeviceCache:
    status = torch.zeros(1, dtype=torch.int32, device=DEV) if with_status else None
    return ssu.DeviceCache(spec.num_slots, spec.nheads, spec.ngroups, spec.ring_len, spec.state_dtype,
                           t["state"], t["scale"], t["x_cache"], t["B_cache"], t["dt_cache"],
                           t["ring_start"], status, spec.headdim, spec.dstate, t.get("recur"), t.get("gscale"))


def out_tensor(step: synth.StepInputs, spec, out_dtype: str):
    dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    return torch.full((step.tokens, spec.nheads, spec.headdim), float("nan"), dtype=dt, device=DEV)


def run_step(dc: ssu.DeviceCache, st: dict, step: synth.StepInputs, out, out_dtype: str, algo: str,
             ws=None, stream=None):
    if algo == "split" and ws is None:
        nbytes = ssu.workspace_size(dc, step.batch, step.T)
        ws = torch.empty(max(nbytes // 4, 1), dtype=torch.float32, device=DEV)
    desc = ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"],
                              st["x"], st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"],
                              out, out_dtype, ws, algo)
    ssu.replay_step(dc, desc, stream)
    return out


def to_f64(out: torch.Tensor) -> np.ndarray:
    return out.detach().to(torch.float64).cpu().numpy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))


def tol_for(state_dtype: str, out_dtype: str) -> float:
    """Parity bounds: 1e-4 (1 + |ref|) for fp32 state with fp32 output,
    2e-2 (1 + |ref|) for bf16 / fp16 / fp8 state or bf16 output."""
    return 1e-4 if (state_dtype == "f32" and out_dtype == "f32") else 2e-2


def fp8_code_agreement(got: np.ndarray, ref: np.ndarray):
    """(fraction equal, max distance in code steps) for e4m3fn codes; +-0 equal."""
    g = got.astype(np.int32)
    r = ref.astype(np.int32)

    def ordinal(c):  # monotone index of the code value: sign-magnitude -> integer line
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)

    og, orf = ordinal(g), ordinal(r)
    same = og == orf
    return float(same.mean()), int(np.max(np.abs(og - orf))) if og.size else 0


def check_cache_after_step(spec, before: synth.CacheArrays, gpu: synth.CacheArrays,
                           ref: synth.CacheArrays):
    """Checkpoint untouched, x/B rings bit-exact with the oracle (appends are
    copies), dt' appends within 1e-6 (1 + |ref|), everything else bit-exact,
    including slot-padding canaries and ring_start."""
    assert np.array_equal(gpu.state, before.state), "checkpoint modified by a replay step"
    assert np.array_equal(gpu.scale, before.scale)
    assert np.array_equal(gpu.x_cache, ref.x_cache), "x ring mismatch"
    assert np.array_equal(gpu.B_cache, ref.B_cache), "B ring mismatch"
    assert np.array_equal(gpu.ring_start, before.ring_start)
    nb = spec.dt_bytes()
    assert np.array_equal(gpu.dt_cache[:, nb:], ref.dt_cache[:, nb:])
    g = gpu.dt_cache[:, :nb].view(np.float32).astype(np.float64)
    r = ref.dt_cache[:, :nb].view(np.float32).astype(np.float64)
    assert rel_err(g, r) <= 1e-6, "dt ring mismatch %g" % rel_err(g, r)
    unchanged = ref.dt_cache[:, :nb].view(np.uint32) == before.dt_cache[:, :nb].view(np.uint32)
    assert np.array_equal(gpu.dt_cache[:, :nb].view(np.uint32)[unchanged],
                          before.dt_cache[:, :nb].view(np.uint32)[unchanged])


def f64_fold(spec, before, slots, k, A, absolute):
    """The oracle's fold of k tokens from `before` in fp64, returned before any
    encoding: [slot] -> [H, P, N].  The starting state is the checkpoint's
    value (the FP16 recurrence checkpoint with separate checkpoints); with
    `absolute`, the fold of |h|, |x| and |B| (every coefficient is >= 0), i.e.
    the sum of the magnitudes of the terms the fold adds up."""
    s64 = synth.CacheSpec(**{**spec.__dict__, "state_dtype": "f64", "state_layout": "rowmajor",
                             "separate": False})
    x, B = before.x_cache.copy(), before.B_cache.copy()
    if absolute:
        x.view(np.uint16)[...] &= 0x7FFF
        B.view(np.uint16)[...] &= 0x7FFF
    c = synth.CacheArrays(s64, np.zeros((spec.num_slots, s64.strides()["state"]), np.uint8),
                          np.zeros((spec.num_slots, s64.strides()["scale"]), np.uint8), x, B,
                          before.dt_cache.copy(), before.ring_start.copy())
    touched = sorted({int(sl) for sl, kk in zip(slots, k) if kk > 0 and 0 < sl < spec.num_slots})
    from oracle import ssu_oracle as O
    for sl in touched:
        h = O.decode_recur(before, sl) if spec.separate else O.decode_state(before, sl)
        c.set_state_logical(sl, np.abs(h) if absolute else h)
    assert O.flush(c, slots, k, A) == 0
    return {sl: c.state_logical(sl) for sl in touched}


# The GPU folds in fp32 with each product's coefficient side split into two
# bf16 parts (relative error <= 2^-18 per term) and fp32 accumulation, so a
# folded value is within FOLD_REL * S of the exact one, S the fold of absolute
# values (f64_fold(..., absolute=True)); 2^-15 leaves a factor > 4 over the
# term-wise bound 2^-18 + (k + 3) 2^-24.
FOLD_REL = 2.0 ** -15


def check_state(spec, gpu, ref, before, touched, fold=None, only=None):
    """Checkpoints after a fold: untouched slots and slot padding bit for bit;
    fp8 codes >= 99.9 % equal and otherwise one code apart; fp8 row scales
    within what the fold error moves the row maximum (fold = (slots, k, A) of
    the fold from `before`; without it 1e-5 relative); other dtypes within
    their relative bounds; nvfp4 as check_nvfp4 (on the folded slots in
    `only`, default all)."""
    if spec.state_dtype == "nvfp4":
        assert fold is not None
        return check_nvfp4(spec, gpu, ref, before, touched, fold, only=only)
    untouched = [s for s in range(spec.num_slots) if s not in touched]
    assert np.array_equal(gpu.state[untouched], before.state[untouched])
    assert np.array_equal(gpu.state[:, spec.state_bytes():], before.state[:, spec.state_bytes():])
    if not touched:
        return
    if spec.state_dtype == "fp8":
        g = np.stack([gpu.state_view(s) for s in touched])
        r = np.stack([ref.state_view(s) for s in touched])
        frac, dist = fp8_code_agreement(g, r)
        assert frac >= 0.999 and dist <= 1, (frac, dist)
        gs = np.stack([gpu.scale_view(s) for s in touched]).astype(np.float64)
        rs = np.stack([ref.scale_view(s) for s in touched]).astype(np.float64)
        if fold is None:
            assert np.max(np.abs(gs - rs) / rs) <= 1e-5
        else:
            s_abs = f64_fold(spec, before, *fold, absolute=True)
            smax = np.stack([s_abs[s].max(axis=-1) for s in touched])  # [slots, H, P]
            tol = FOLD_REL * smax.reshape(gs.shape) / 448.0 + 2.0 ** -22 * rs
            assert np.all(np.abs(gs - rs) <= tol), float(np.max(np.abs(gs - rs) - tol))
    else:
        g = np.stack([_decode_state(gpu, s) for s in touched])
        r = np.stack([_decode_state(ref, s) for s in touched])
        assert rel_err(g, r) <= (1e-4 if spec.state_dtype == "f32" else 2e-2)


def state_propagation_bound(spec, step, k, gpu, ref_cache):
    """Per output element, the most the readout can move between the GPU's
    re-encoded checkpoint and the oracle's: the readout of token i is
    beta_i C_i.h with beta_i = exp(cumA) <= 1 (A < 0, dt' >= 0), so the two
    differ by at most sum_n |C_i[n]| |h_gpu[p, n] - h_ref[p, n]|.  The state
    check bounds those differences (fp8: one code in at most 0.1 % of the
    elements), and this lets the output check accept the readout of any
    checkpoint that passes it."""
    extra = np.zeros((step.tokens, spec.nheads, spec.headdim))
    hpg = spec.nheads // spec.ngroups
    C = bf16_bits_to_f64(step.C)
    for b in range(step.batch):
        slot = int(step.slot_idx[b])
        if k[b] <= 0 or not 0 < slot < spec.num_slots:
            continue
        bos = int(step.cu_seqlens[b]) if step.cu_seqlens is not None else b * step.T
        tb = (int(step.cu_seqlens[b + 1]) - bos) if step.cu_seqlens is not None else step.T
        dh = np.abs(_decode_state(gpu, slot) - _decode_state(ref_cache, slot))  # [H, P, N]
        for h in range(spec.nheads):
            extra[bos:bos + tb, h, :] = np.abs(C[bos:bos + tb, h // hpg]) @ dh[h].T
    return extra


def fused_plain_reference(spec, step, k, gpu):
    """The oracle's plain step with pnat - k live tokens run on the GPU's own
    cache after a fused call (its re-encoded checkpoints and advanced ring
    starts; the live tokens it reads are not touched by the call's appends,
    which land after them).  An entry whose k the call rejected is read as
    padding (zero rows)."""
    from oracle import ssu_oracle as O
    import dataclasses
    slots = np.asarray(step.slot_idx, np.int32).copy()
    pnat = np.asarray(step.pnat, np.int32).copy()
    for b in range(step.batch):
        if 0 <= k[b] <= pnat[b]:
            pnat[b] -= k[b]
        else:
            slots[b] = 0
    ref, _ = O.replay_step(gpu.copy(), dataclasses.replace(step, slot_idx=slots, pnat=pnat))
    return ref


def check_fused_outputs(spec, step, k, out, gpu, ref, ref_cache, out_dtype, rows=None):
    """Outputs of a fused flush-in-step, two ways.
    1. Against the oracle's plain step on the GPU's own post-fold checkpoint
       (fused_plain_reference), at the plain bound of the output and state
       dtypes: the readout itself, with no allowance for the fold.
    2. Against the oracle's own flush-then-step composition, where the GPU
       reads out from its re-encoded checkpoint and the oracle from its own:
       the plain bound plus what the state differences the state check
       accepts move the readout (state_propagation_bound, times |silu(z)|
       for a gated step).
    `rows`: output rows of `out` that belong to `step` (a sampled subset)."""
    got = to_f64(out) if rows is None else to_f64(out)[rows]
    tol = tol_for(spec.state_dtype, out_dtype)
    plain = fused_plain_reference(spec, step, k, gpu)
    err = rel_err(got, plain)
    assert err <= tol, "fused readout vs the oracle's step on the GPU checkpoint: rel err %g > %g" % (err, tol)
    extra = state_propagation_bound(spec, step, k, gpu, ref_cache)
    if getattr(step, "z", None) is not None:
        zv = bf16_bits_to_f64(step.z)
        extra = extra * np.abs(zv / (1.0 + np.exp(-zv)))
    excess = np.abs(got - ref) - tol * (1.0 + np.abs(ref)) - extra
    assert np.all(excess <= 1e-12 * (1.0 + np.abs(ref))), "composition: max excess %g" % np.max(excess)
    return err


def bf16_bits_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def _decode_state(cache, slot):
    from oracle import ssu_oracle as O
    return O.decode_state(cache, slot)


def _f16_ordinal(bits):
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_recur(spec, gpu, before, slots, k, A, seed, min_equal=0.98, bits_slot=None, only=None):
    """Recurrence checkpoints after a fold of k tokens from `before`:
    untouched slots and slot padding bit for bit, folded ones bracketed by
    stochastic rounding of the exact fold +- the fp32 error bound (`only`:
    the folded slots to bracket, default all).  The random bits of cache slot
    s are those of slot bits_slot[s] (the slot the GPU saw, when `before` is
    a renumbered subset)."""
    from oracle import ssu_oracle as O
    touched = sorted({int(sl) for sl, kk in zip(slots, k) if kk > 0 and 0 < sl < spec.num_slots})
    untouched = [sl for sl in range(spec.num_slots) if sl not in touched]
    assert np.array_equal(gpu.recur[untouched], before.recur[untouched])
    nb = spec.recur_bytes()
    assert np.array_equal(gpu.recur[:, nb:], before.recur[:, nb:])  # slot padding
    if only is not None:
        touched = [sl for sl in touched if sl in set(only)]
    if not touched:
        return
    slots, k = _fold_subset(slots, k, touched)
    v_ref = f64_fold(spec, before, slots, k, A, absolute=False)
    s_abs = f64_fold(spec, before, slots, k, A, absolute=True)
    P, N = spec.headdim, spec.dstate
    equal = total = 0
    for sl in touched:
        bs = sl if bits_slot is None else bits_slot[sl]
        u = np.stack([O.sr_bits(seed, bs, h, P * N).reshape(P, N) for h in range(spec.nheads)])
        v, S = v_ref[sl], s_abs[sl]
        E = FOLD_REL * S + 2.0 ** -23 * np.abs(v)
        lo = _f16_ordinal(O.sr_f16(v - E, u))
        hi = _f16_ordinal(O.sr_f16(v + E, u))
        g = _f16_ordinal(gpu.recur_logical(sl))
        bad = (g < lo) | (g > hi)
        assert not bad.any(), "slot %d: %d values outside the bracket, first at %s" % (
            sl, int(bad.sum()), np.argwhere(bad)[0])
        equal += int((g == _f16_ordinal(O.sr_f16(v, u))).sum())
        total += g.size
    assert equal >= min_equal * total, equal / total




def _e4m3(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def block_scale_values(cache, slot):
    """The e4m3 block-scale values of one slot as [H, P, N / 16], read with
    the tiled layout (lane l = 16 q + m of row 16 rb + m: byte l * 8 + rb * 2
    + j for the block of values 32 q + 16 j .. + 15)."""
    raw = cache.scale_view(slot)  # [H, 512] bytes in storage order
    p = np.arange(64)[:, None]
    blk = np.arange(8)[None, :]
    rb, m, q, j = p // 16, p % 16, blk // 2, blk % 2
    idx = (16 * q + m) * 8 + rb * 2 + j
    return _e4m3(raw[:, idx])


def _ordinal(codes, sign_bit):
    """Monotone index of sign-magnitude codes on the value line (+-0 equal)."""
    c = codes.astype(np.int32)
    mag = c & (sign_bit - 1)
    return np.where(c & sign_bit, -mag, mag)


def _fold_subset(slots, k, keep):
    """The fold restricted to the slots in `keep` (others fold nothing)."""
    keep = set(int(x) for x in keep)
    k2 = np.array([kk if int(sl) in keep else 0 for sl, kk in zip(slots, k)], np.int32)
    return np.asarray(slots, np.int32), k2


def check_nvfp4(spec, gpu, ref, before, touched, fold, min_equal=0.999, only=None):
    """NVFP4 read checkpoints after a fold of `fold` = (slots, k, A) from
    `before`.  Untouched slots bit for bit.  The slot scale (word 0) and the
    head maxima (words 1 + h) within what the fold error moves a maximum.
    Every decoded value within one element step (e4m3 block scale * g) of
    the exact fold plus the fold bound, or saturated at 6 block-scale units
    where a subnormal block scale rounded below a sixth of its block maximum.
    Codes and block scales as the fp8 rule for codes: >= 99.9 % equal to the
    oracle's, the rest one code apart (the GPU encodes its own fp32 fold,
    within FOLD_REL * S of the exact one, so a code can differ only where a
    value lies that close to a rounding midpoint)."""
    from oracle import ssu_oracle as O
    untouched = [s for s in range(spec.num_slots) if s not in touched]
    for f in ("state", "scale", "gscale"):
        assert np.array_equal(getattr(gpu, f)[untouched], getattr(before, f)[untouched]), f
    if only is not None:
        touched = [sl for sl in touched if sl in set(only)]
        fold = (*_fold_subset(fold[0], fold[1], touched), fold[2])
    v_ex = f64_fold(spec, before, *fold, absolute=False)
    s_abs = f64_fold(spec, before, *fold, absolute=True)
    equal = total = sf_equal = sf_total = 0
    worst = 0
    for sl in touched:
        wg = gpu.gscale_view(sl).astype(np.float64)
        wr = ref.gscale_view(sl).astype(np.float64)
        smax = s_abs[sl].reshape(spec.nheads, -1).max(axis=1)  # per head
        assert np.all(np.abs(wg[1:] - wr[1:]) <= FOLD_REL * smax + 2.0 ** -23 * wr[1:]), (sl, wg[1:], wr[1:])
        gg, gr = wg[0], wr[0]
        assert abs(gg - gr) <= FOLD_REL * smax.max() / 2688.0 + 2.0 ** -22 * gr, (sl, gg, gr)
        dec_g, dec_r = O.decode_state(gpu, sl), O.decode_state(ref, sl)
        es = block_scale_values(gpu, sl) * gg  # [H, P, 8]
        es = np.repeat(np.where(es == 0, 6.0 * gg * 2.0 ** -10, es), 16, axis=2)
        err_fold = FOLD_REL * s_abs[sl]
        sat = np.maximum(np.abs(v_ex[sl]) + err_fold - 6.0 * es, 0.0)
        over = np.abs(dec_g - v_ex[sl]) - (es + sat + err_fold + 1e-30)
        assert np.all(over <= 0), (sl, float(np.max(over)))
        cg, cr = gpu.state_view(sl), ref.state_view(sl)
        for sh in (0, 4):
            og, orf = _ordinal((cg >> sh) & 15, 8), _ordinal((cr >> sh) & 15, 8)
            equal += int((og == orf).sum())
            total += og.size
            worst = max(worst, int(np.max(np.abs(og - orf))))
        sg, sr = _ordinal(gpu.scale_view(sl), 0x80), _ordinal(ref.scale_view(sl), 0x80)
        sf_equal += int((sg == sr).sum())
        sf_total += sg.size
        worst = max(worst, int(np.max(np.abs(sg - sr))))
    print("nvfp4 codes equal %.6f, block scales equal %.6f, max code distance %d" % (
        equal / max(total, 1), sf_equal / max(sf_total, 1), worst), flush=True)
    assert equal >= min_equal * total, equal / total
    assert sf_equal >= min_equal * sf_total, sf_equal / sf_total
    assert worst <= 1, worst
