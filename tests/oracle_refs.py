"""Independent fp64 restatements used to pin the oracle (test-only helpers).

Each function here computes a quantity the oracle also computes, but by a
different route (a closed form, a matrix identity, arbitrary precision), so
that a slip in the oracle's sequential code shows up as a mismatch.  Nothing
here is shared with the oracle's C code.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 through torch's own bf16 type."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16)
    return t.to(torch.float64).numpy()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def state_f64(cache, slot) -> np.ndarray:
    """Checkpoint value [H, P, N] decoded through torch's dtypes."""
    s = cache.spec
    raw = cache.state_logical(slot)
    if s.state_dtype in ("f32", "f64"):
        return raw.astype(np.float64)
    if s.state_dtype == "bf16":
        return bf16_to_f64(raw)
    if s.state_dtype == "f16":
        return f16_to_f64(raw)
    return e4m3_to_f64(raw) * cache.scale_view(slot).astype(np.float64)[:, :, None]


def softplus_torch(v: np.ndarray) -> np.ndarray:
    return torch.nn.functional.softplus(torch.from_numpy(np.asarray(v, np.float64)),
                                        beta=1.0, threshold=20.0).numpy()


def sequence(cache, step, b, h):
    """The combined sequence of entry b, head h, gathered by the ring contract.

    Returns dict with dtp [S], x [S, P], B [S, N], C [T_b, N], xnew [T_b, P],
    pnat, Tb, bos.  Live token j is ring entry (ring_start + j) mod L; new
    token i follows it at combined index pnat + i.
    """
    s = cache.spec
    L, HPG = s.ring_len, s.nheads // s.ngroups
    g = h // HPG
    slot = int(step.slot_idx[b])
    p = int(step.pnat[b])
    if step.cu_seqlens is not None:
        bos = int(step.cu_seqlens[b])
        Tb = int(step.cu_seqlens[b + 1]) - bos
    else:
        bos, Tb = b * step.T, step.T
    r = int(cache.ring_start[slot])
    pos = [(r + j) % L for j in range(p)]
    xr = bf16_to_f64(cache.x_view(slot)[h][pos]) if p else np.zeros((0, s.headdim))
    Br = bf16_to_f64(cache.B_view(slot)[g][pos]) if p else np.zeros((0, s.dstate))
    dr = cache.dt_view(slot)[h][pos].astype(np.float64) if p else np.zeros(0)
    toks = np.arange(bos, bos + Tb)
    xn = bf16_to_f64(step.x[toks, h])
    Bn = bf16_to_f64(step.B[toks, g])
    Cn = bf16_to_f64(step.C[toks, g])
    raw = step.dt[toks, h].astype(np.float64) + float(step.dt_bias[h])
    dn = softplus_torch(raw) if getattr(step, "dt_softplus", True) else raw
    return dict(dtp=np.concatenate([dr, dn]), x=np.concatenate([xr, xn]),
                B=np.concatenate([Br, Bn]), C=Cn, xnew=xn, pnat=p, Tb=Tb, bos=bos,
                slot=slot, g=g)


def closed_form_outputs(h0, A, D, seq):
    """y_t = C_t (e^{cumA_t} h0) + sum_{s<=t} e^{cumA_t - cumA_s} dt'_s (C_t.B_s) x_s + D x_t.

    h0 [P, N]; A, D scalars; seq from `sequence`.  Returns [T_b, P].
    """
    p, Tb = seq["pnat"], seq["Tb"]
    cum = np.cumsum(A * seq["dtp"])  # inclusive prefix of the decay exponent
    Y = np.zeros((Tb, h0.shape[0]))
    for i in range(Tb):
        t = p + i
        y = np.exp(cum[t]) * (h0 @ seq["C"][i])
        for s_ in range(t + 1):
            w = np.exp(cum[t] - cum[s_]) * seq["dtp"][s_] * float(seq["C"][i] @ seq["B"][s_])
            y = y + w * seq["x"][s_]
        Y[i] = y + D * seq["xnew"][i]
    return Y


def closed_form_state(h0, A, dtp, x, B):
    """h_k = e^{cumA_{k-1}} h0 + sum_{s<k} e^{cumA_{k-1} - cumA_s} dt'_s x_s B_s^T."""
    k = len(dtp)
    if k == 0:
        return h0.copy()
    cum = np.cumsum(A * np.asarray(dtp))
    coef = np.exp(cum[-1] - cum) * dtp
    return np.exp(cum[-1]) * h0 + np.einsum("s,sp,sn->pn", coef, x, B)
