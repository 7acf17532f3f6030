"""Device plumbing for the synthetic inputs: upload host arrays, draw full-size
caches directly on the GPU (same value laws as `workloads`), and copy a
subset of slots back to the host for sampled oracle checks.

Torch only moves and draws data here; nothing of the method is computed.
"""
from __future__ import annotations

import math
from typing import Dict, Sequence

import numpy as np
import torch

from .workloads import CANARY, CacheArrays, CacheSpec, StepInputs

CACHE_FIELDS = ("state", "scale", "x_cache", "B_cache", "dt_cache")
_STRIDE_KEY = {"state": "state", "scale": "scale", "x_cache": "x", "B_cache": "B", "dt_cache": "dt"}


def upload_cache(cache: CacheArrays, device) -> Dict[str, torch.Tensor]:
    t = {f: torch.from_numpy(getattr(cache, f)).to(device) for f in CACHE_FIELDS}
    t["ring_start"] = torch.from_numpy(cache.ring_start).to(device)
    t["recur"] = None if cache.recur is None else torch.from_numpy(cache.recur).to(device)
    t["gscale"] = None if cache.gscale is None else torch.from_numpy(cache.gscale).to(device)
    return t


def _opt(t, key, idx=None):
    a = t.get(key)
    if a is None:
        return None
    return (a if idx is None else a.index_select(0, idx)).cpu().numpy()


def download_cache(spec: CacheSpec, t: Dict[str, torch.Tensor]) -> CacheArrays:
    return CacheArrays(spec, *(t[f].cpu().numpy() for f in CACHE_FIELDS),
                       t["ring_start"].cpu().numpy(), _opt(t, "recur"), _opt(t, "gscale"))


def download_subset(spec: CacheSpec, t: Dict[str, torch.Tensor], slots: Sequence[int]):
    """Host cache holding slot pages [0] + slots (renumbered 1..len(slots)).

    Returns (CacheArrays with num_slots = len(slots) + 1, mapping old -> new).
    """
    slots = [int(s) for s in slots]
    idx = torch.tensor([0] + slots, dtype=torch.long, device=t["state"].device)
    sub = CacheSpec(**{**spec.__dict__, "num_slots": len(slots) + 1})
    arrs = [t[f].index_select(0, idx).cpu().numpy() for f in CACHE_FIELDS]
    rs = t["ring_start"].index_select(0, idx).cpu().numpy()
    return (CacheArrays(sub, *arrs, rs, _opt(t, "recur", idx), _opt(t, "gscale", idx)),
            {s: i + 1 for i, s in enumerate(slots)})


def _bf16_bytes(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).view(torch.uint8)


def make_cache_device(spec: CacheSpec, seed: int, device, h0_std: float = 0.1,
                      chunk_slots: int = 64) -> Dict[str, torch.Tensor]:
    """A full cache drawn on the device (value laws of workloads.make_cache)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    S, H, G, P, N, L = (spec.num_slots, spec.nheads, spec.ngroups, spec.headdim, spec.dstate,
                        spec.ring_len)
    st = spec.strides()
    t = {f: torch.full((S, st[_STRIDE_KEY[f]]), CANARY, dtype=torch.uint8, device=device)
         for f in CACHE_FIELDS}
    t["gscale"] = (torch.full((S, st["gscale"]), CANARY, dtype=torch.uint8, device=device)
                   if "gscale" in st else None)
    dt = spec.state_dtype
    for s0 in range(0, S, chunk_slots):
        n = min(chunk_slots, S - s0)
        sl = slice(s0, s0 + n)
        if dt == "nvfp4":  # the law of workloads.random_nvfp4
            t["state"][sl, : spec.state_bytes()] = torch.randint(
                0, 256, (n, H * P * N // 2), generator=g, device=device, dtype=torch.int32).to(torch.uint8)
            e = torch.randint(5, 9, (n, H * P * N // 16), generator=g, device=device, dtype=torch.int32)
            m = torch.randint(0, 8, (n, H * P * N // 16), generator=g, device=device, dtype=torch.int32)
            t["scale"][sl, : spec.scale_bytes()] = (e * 8 + m).to(torch.uint8)
            gs = (h0_std / 3.0) * (0.5 + torch.rand(n, 1, generator=g, device=device))
            words = torch.cat([gs, (gs * 2688.0).expand(n, H)], dim=1).contiguous()
            t["gscale"][sl, : spec.gscale_bytes()] = words.view(torch.uint8).reshape(n, -1)
        elif dt == "fp8":
            codes = (torch.randn(n, H, P, N, generator=g, device=device) * 32.0).clamp(-448, 448)
            t["state"][sl, : spec.state_bytes()] = codes.to(torch.float8_e4m3fn).view(
                torch.uint8).reshape(n, -1)
            sc = (h0_std / 32.0) * (0.5 + torch.rand(n, H, P, generator=g, device=device))
            t["scale"][sl, : spec.scale_bytes()] = sc.view(torch.uint8).reshape(n, -1)
        else:
            h0 = torch.randn(n, H, P, N, generator=g, device=device) * h0_std
            tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16,
                   "f64": torch.float64}[dt]
            t["state"][sl, : spec.state_bytes()] = h0.to(tdt).view(torch.uint8).reshape(n, -1)
        t["x_cache"][sl, : spec.x_bytes()] = _bf16_bytes(
            torch.randn(n, H, L, P, generator=g, device=device)).reshape(n, -1)
        t["B_cache"][sl, : spec.B_bytes()] = _bf16_bytes(
            torch.randn(n, G, L, N, generator=g, device=device)).reshape(n, -1)
        lo, hi = math.log(0.004), math.log(0.5)
        d = torch.exp(lo + (hi - lo) * torch.rand(n, H, L, generator=g, device=device))
        t["dt_cache"][sl, : spec.dt_bytes()] = d.view(torch.uint8).reshape(n, -1)
    t["ring_start"] = torch.randint(0, L, (S,), generator=g, device=device, dtype=torch.int32)
    t["recur"] = None
    if spec.separate:
        t["recur"] = torch.full((S, st["recur"]), CANARY, dtype=torch.uint8, device=device)
        for s0 in range(0, S, chunk_slots):
            n = min(chunk_slots, S - s0)
            h0 = torch.randn(n, H, P, N, generator=g, device=device) * h0_std
            t["recur"][s0:s0 + n, : spec.recur_bytes()] = h0.to(torch.float16).view(torch.uint8).reshape(n, -1)
    return t


def upload_step(step: StepInputs, device) -> Dict[str, torch.Tensor]:
    def u16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)

    t = dict(
        slot_idx=torch.from_numpy(step.slot_idx).to(device),
        pnat=torch.from_numpy(step.pnat).to(device),
        cu_seqlens=None if step.cu_seqlens is None else torch.from_numpy(step.cu_seqlens).to(device),
        x=u16(step.x), B=u16(step.B), C=u16(step.C),
        dt=torch.from_numpy(step.dt).to(device),
        A=torch.from_numpy(step.A).to(device), D=torch.from_numpy(step.D).to(device),
        dt_bias=torch.from_numpy(step.dt_bias).to(device),
        z=None if step.z is None else u16(step.z),
    )
    return t


def subset_step(step: StepInputs, entries: Sequence[int], slot_map) -> StepInputs:
    """The listed entries of a step as their own step, slots renumbered by slot_map
    (padding / unknown slots map to 0)."""
    entries = [int(b) for b in entries]
    rows, cu = [], [0]
    for b in entries:
        if step.cu_seqlens is not None:
            lo, hi = int(step.cu_seqlens[b]), int(step.cu_seqlens[b + 1])
        else:
            lo, hi = b * step.T, (b + 1) * step.T
        rows.extend(range(lo, hi))
        cu.append(cu[-1] + hi - lo)
    rows = np.asarray(rows, np.int64)
    slots = np.array([slot_map.get(int(step.slot_idx[b]), 0) for b in entries], np.int32)
    return StepInputs(len(entries), step.T, slots, step.pnat[entries].astype(np.int32),
                      np.asarray(cu, np.int32) if step.cu_seqlens is not None else None,
                      step.x[rows], step.B[rows], step.C[rows], step.dt[rows],
                      step.A, step.D, step.dt_bias, None if step.z is None else step.z[rows],
                      step.dt_softplus)
