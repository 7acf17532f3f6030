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


def check_state(spec, gpu, ref, before, touched, fold=None):
    """Checkpoints after a fold: untouched slots and slot padding bit for bit;
    fp8 codes >= 99.9 % equal and otherwise one code apart; fp8 row scales
    within what the fold error moves the row maximum (fold = (slots, k, A) of
    the fold from `before`; without it 1e-5 relative); other dtypes within
    their relative bounds."""
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


def bf16_bits_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def _decode_state(cache, slot):
    from oracle import ssu_oracle as O
    return O.decode_state(cache, slot)
