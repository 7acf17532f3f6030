"""Seeded synthetic inputs for the ReplaySSM step and flush.

This module draws random numbers into the cache and step layouts and nothing
else: it holds none of the method's arithmetic (no softplus, no decay, no
encoding rule), so that the GPU library and the CPU oracle, which both read
these arrays, cannot share a mistake through it.  Casting a random fp32 sample
to bf16 / fp16 / fp8 is done with PyTorch's own CPU casts.

Cache layout (one slot = one request), matching the ring-buffer cache contract
of the FlashInfer checkpointing-SSU page (Description, item 2) and the vLLM
replayssm_cutedsl page (slot 0 reserved for padding, padding allowed between
slot pages):

    state     [slot][H][P][N]   state dtype
    scale     [slot][H][P]      f32 (fp8 state only)
    x_cache   [slot][H][L][P]   bf16
    B_cache   [slot][G][L][N]   bf16
    dt_cache  [slot][H][L]      f32 (holds dt' = softplus(dt + dt_bias))
    ring_start[slot]            i32

Every per-slot tensor is stored as a byte array [num_slots, stride] whose
stride is the packed size plus `slot_pad` bytes; pad bytes hold a canary.

Value laws (the synthetic workloads' recipe): x, B, C ~ N(0, 1) in bf16;
dt ~ N(0, 0.5^2); dt_bias ~ U(-4, -2); A = -exp(U(0, ln 16)); D ~ N(0, 1);
checkpoint h0 ~ N(0, 0.1^2).  Ring dt' values are drawn log-uniform on
[0.004, 0.5], the range softplus(dt + dt_bias) covers under the laws above.
An fp8 checkpoint is drawn as random e4m3 codes (a N(0, 32^2) sample cast to
e4m3fn) with a per-row scale 0.1/32 * U(0.5, 1.5), which gives h0 of about the
same spread.  All L ring entries (live and dead) hold random data, so reading
a wrong entry changes the result.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

DTYPES = ("f32", "bf16", "f16", "fp8", "f64", "nvfp4")
ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1, "f64": 8, "nvfp4": 0.5}
CANARY = 0xA5


def _round16(n: int) -> int:
    return (n + 15) // 16 * 16


@dataclasses.dataclass
class CacheSpec:
    num_slots: int
    nheads: int
    ngroups: int
    headdim: int = 64
    dstate: int = 128
    ring_len: int = 16
    state_dtype: str = "bf16"
    slot_pad: int = 0  # bytes appended to every per-slot stride
    state_layout: str = ""  # "tiled" (the library's layout, 64 x 128 heads) or "rowmajor"
    separate: bool = False  # an FP16 recurrence checkpoint next to the read checkpoint

    def __post_init__(self):
        assert self.state_dtype in DTYPES
        assert self.nheads % self.ngroups == 0
        if not self.state_layout:
            tiled_ok = (self.headdim, self.dstate) == (64, 128) and self.state_dtype != "f64"
            self.state_layout = "tiled" if tiled_ok else "rowmajor"
        assert self.state_layout in ("tiled", "rowmajor")

    # packed per-slot byte sizes
    def state_bytes(self):
        return int(self.nheads * self.headdim * self.dstate * ELEM_BYTES[self.state_dtype])

    def recur_bytes(self):
        return self.nheads * self.headdim * self.dstate * 2

    def scale_bytes(self):
        """fp8: an f32 scale per row; nvfp4: an e4m3 scale per 16 values."""
        if self.state_dtype == "nvfp4":
            return self.nheads * self.headdim * self.dstate // 16
        return self.nheads * self.headdim * 4

    def gscale_bytes(self):
        """nvfp4: f32 words [1 + H]: the slot's second-level scale, then the
        largest |value| of each head at its last encode."""
        return (1 + self.nheads) * 4

    def x_bytes(self):
        return self.nheads * self.ring_len * self.headdim * 2

    def B_bytes(self):
        return self.ngroups * self.ring_len * self.dstate * 2

    def dt_bytes(self):
        return self.nheads * self.ring_len * 4

    def strides(self):
        """Per-slot byte strides (packed size rounded to 16 B, plus the pad)."""
        p = self.slot_pad
        d = dict(
            state=_round16(self.state_bytes()) + p,
            scale=_round16(self.scale_bytes()) + p,
            x=_round16(self.x_bytes()) + p,
            B=_round16(self.B_bytes()) + p,
            dt=_round16(self.dt_bytes()) + p,
        )
        if self.separate:
            d["recur"] = _round16(self.recur_bytes()) + p
        if self.state_dtype == "nvfp4":
            d["gscale"] = _round16(self.gscale_bytes()) + p
        return d


def tiled_index(eb: int) -> np.ndarray:
    """Storage element index of each logical element (p, n) of a 64 x 128 head
    in the tiled layout, as an array [64, 128].

    Rows come in blocks of 16 (rb = p // 16, m = p % 16), each row in four
    quarters of 32 values (q = n // 32, t = n % 32); quarter q of row p belongs
    to lane l = 16 q + m and is cut into 16-byte chunks of ce = 16 // eb values;
    chunk u = t // ce of lane l is the (64 u + l)-th chunk of the row block.
    """
    ce = 16 // eb
    p = np.arange(64)[:, None]
    n = np.arange(128)[None, :]
    rb, m, q, t = p // 16, p % 16, n // 32, n % 32
    lane = 16 * q + m
    return rb * 2048 + (t // ce) * (64 * ce) + lane * ce + t % ce


@dataclasses.dataclass
class CacheArrays:
    spec: CacheSpec
    state: np.ndarray  # uint8 [num_slots, stride]
    scale: np.ndarray
    x_cache: np.ndarray
    B_cache: np.ndarray
    dt_cache: np.ndarray
    ring_start: np.ndarray  # int32 [num_slots]
    recur: Optional[np.ndarray] = None  # uint8 [num_slots, stride]: FP16 recurrence checkpoint
    gscale: Optional[np.ndarray] = None  # uint8 [num_slots, stride]: nvfp4 second-level scales

    def copy(self) -> "CacheArrays":
        return CacheArrays(self.spec, *(a.copy() for a in (
            self.state, self.scale, self.x_cache, self.B_cache, self.dt_cache,
            self.ring_start)), None if self.recur is None else self.recur.copy(),
            None if self.gscale is None else self.gscale.copy())

    def recur_view(self, slot):
        """Recurrence checkpoint (fp16 bits) of one slot in storage order, [H, P * N]."""
        s = self.spec
        return self.recur[slot, : s.recur_bytes()].view(np.uint16).reshape(s.nheads, s.headdim * s.dstate)

    def recur_logical(self, slot):
        """Recurrence checkpoint (fp16 bits) of one slot as [H, P, N] (a copy)."""
        s = self.spec
        v = self.recur_view(slot)
        if s.state_layout == "rowmajor":
            return v.reshape(s.nheads, s.headdim, s.dstate).copy()
        return v[:, tiled_index(2)]

    # typed views of the packed part of one slot (for tests)
    def _state_np_dtype(self):
        return {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16,
                "fp8": np.uint8, "f64": np.float64, "nvfp4": np.uint8}[self.spec.state_dtype]

    def state_view(self, slot):
        """Checkpoint elements of one slot in storage order, [H, P * N] (a view)."""
        s = self.spec
        raw = self.state[slot, : s.state_bytes()]
        return raw.view(self._state_np_dtype()).reshape(s.nheads, -1)

    def state_logical(self, slot):
        """Checkpoint elements of one slot as [H, P, N] (a copy, logical order)."""
        s = self.spec
        if s.state_dtype == "nvfp4":
            raise NotImplementedError("nvfp4 packs two codes per byte; decode with the oracle")
        v = self.state_view(slot)
        if s.state_layout == "rowmajor":
            return v.reshape(s.nheads, s.headdim, s.dstate).copy()
        return v[:, tiled_index(ELEM_BYTES[s.state_dtype])]

    def set_state_logical(self, slot, values):
        """Write [H, P, N] logical elements into one slot's storage."""
        s = self.spec
        v = self.state_view(slot)
        values = np.asarray(values, self._state_np_dtype()).reshape(s.nheads, s.headdim, s.dstate)
        if s.state_layout == "rowmajor":
            v[:] = values.reshape(s.nheads, -1)
        else:
            v[:, tiled_index(ELEM_BYTES[s.state_dtype])] = values

    def scale_view(self, slot):
        s = self.spec
        if s.state_dtype == "nvfp4":  # e4m3 block scales in storage order
            return self.scale[slot, : s.scale_bytes()].reshape(s.nheads, -1)
        return self.scale[slot, : s.scale_bytes()].view(np.float32).reshape(s.nheads, s.headdim)

    def gscale_view(self, slot):
        s = self.spec
        return self.gscale[slot, : s.gscale_bytes()].view(np.float32)

    def x_view(self, slot):
        s = self.spec
        return self.x_cache[slot, : s.x_bytes()].view(np.uint16).reshape(
            s.nheads, s.ring_len, s.headdim)

    def B_view(self, slot):
        s = self.spec
        return self.B_cache[slot, : s.B_bytes()].view(np.uint16).reshape(
            s.ngroups, s.ring_len, s.dstate)

    def dt_view(self, slot):
        s = self.spec
        return self.dt_cache[slot, : s.dt_bytes()].view(np.float32).reshape(s.nheads, s.ring_len)


@dataclasses.dataclass
class StepInputs:
    batch: int
    T: int  # tokens per entry, or the maximum per entry when varlen
    slot_idx: np.ndarray  # int32 [batch]
    pnat: np.ndarray  # int32 [batch]
    cu_seqlens: Optional[np.ndarray]  # int32 [batch+1] or None
    x: np.ndarray  # uint16 (bf16 bits) [tokens, H, P]
    B: np.ndarray  # uint16 [tokens, G, N]
    C: np.ndarray  # uint16 [tokens, G, N]
    dt: np.ndarray  # f32 [tokens, H]
    A: np.ndarray  # f32 [H]
    D: np.ndarray  # f32 [H]
    dt_bias: np.ndarray  # f32 [H]
    z: Optional[np.ndarray] = None  # uint16 (bf16 bits) [tokens, H, P]: output gate, or None
    dt_softplus: bool = True  # False: dt' = dt + dt_bias (no softplus)

    @property
    def tokens(self) -> int:
        return int(self.cu_seqlens[-1]) if self.cu_seqlens is not None else self.batch * self.T


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def _bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def _fill_slots(arr: np.ndarray, packed: np.ndarray):
    """Write `packed` (shape [num_slots, nbytes], uint8) into the slot pages."""
    arr[:, : packed.shape[1]] = packed


def random_nvfp4(n: int, H: int, P: int, N: int, g: torch.Generator, h0_std: float = 0.1):
    """Random nvfp4 checkpoints: every code byte uniform (all 16 e2m1 codes in
    both nibbles), block-scale codes with exponent field 5..8 and a random
    mantissa (e4m3 values 0.25 .. 3.75), one second-level scale per slot
    h0_std / 3 * U(0.5, 1.5), head maxima words 2688 times it: codes, block
    scales and scale words as byte arrays [n, ...]."""
    codes = torch.randint(0, 256, (n, H * P * N // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    e = torch.randint(5, 9, (n, H * P * N // 16), generator=g, dtype=torch.int32)
    m = torch.randint(0, 8, (n, H * P * N // 16), generator=g, dtype=torch.int32)
    sf = (e * 8 + m).to(torch.uint8)
    gs = (h0_std / 3.0) * (0.5 + torch.rand(n, 1, generator=g))
    words = torch.cat([gs, (gs * 2688.0).expand(n, H)], dim=1)
    return codes.numpy(), sf.numpy(), words.to(torch.float32).numpy().view(np.uint8).reshape(n, -1)


def random_state_bytes(spec: CacheSpec, n: int, g: torch.Generator, h0_std: float = 0.1):
    """Random checkpoints for n slots: (state bytes [n, state_bytes], scale bytes)."""
    H, P, N = spec.nheads, spec.headdim, spec.dstate
    dt = spec.state_dtype
    scale = np.zeros((n, H * P * 4), np.uint8)
    assert dt != "nvfp4", "nvfp4 checkpoints come from random_nvfp4"
    if dt == "fp8":
        codes = (torch.randn(n, H, P, N, generator=g) * 32.0).clamp(-448, 448)
        codes = codes.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        sc = (h0_std / 32.0) * (0.5 + torch.rand(n, H, P, generator=g))
        scale = sc.to(torch.float32).numpy().view(np.uint8).reshape(n, -1)
        return codes.reshape(n, -1), scale
    h0 = torch.randn(n, H, P, N, generator=g, dtype=torch.float64) * h0_std
    if dt == "f64":
        raw = h0.numpy().view(np.uint8)
    elif dt == "f32":
        raw = h0.to(torch.float32).numpy().view(np.uint8)
    elif dt == "bf16":
        raw = _bf16_bits(h0.to(torch.float32)).view(np.uint8)
    else:
        raw = _f16_bits(h0.to(torch.float32)).view(np.uint8)
    return raw.reshape(n, -1), scale


def make_cache(spec: CacheSpec, seed: int, h0_std: float = 0.1) -> CacheArrays:
    """A cache with random checkpoints, random rings and random ring_start."""
    g = _gen(seed)
    S, H, G, P, N, L = (spec.num_slots, spec.nheads, spec.ngroups, spec.headdim,
                        spec.dstate, spec.ring_len)
    st = spec.strides()
    arrs = {k: np.full((S, st[k]), CANARY, np.uint8) for k in st}
    gscale = None
    if spec.state_dtype == "nvfp4":
        state, scale, gs = random_nvfp4(S, H, P, N, g, h0_std)
        gscale = arrs["gscale"]
        _fill_slots(gscale, gs)
    else:
        state, scale = random_state_bytes(spec, S, g, h0_std)
    _fill_slots(arrs["state"], state)
    if spec.state_dtype in ("fp8", "nvfp4"):
        _fill_slots(arrs["scale"], scale)
    xr = _bf16_bits(torch.randn(S, H, L, P, generator=g)).view(np.uint8).reshape(S, -1)
    Br = _bf16_bits(torch.randn(S, G, L, N, generator=g)).view(np.uint8).reshape(S, -1)
    lo, hi = math.log(0.004), math.log(0.5)
    dtr = torch.exp(lo + (hi - lo) * torch.rand(S, H, L, generator=g, dtype=torch.float64))
    dtr = dtr.to(torch.float32).numpy().view(np.uint8).reshape(S, -1)
    _fill_slots(arrs["x"], xr)
    _fill_slots(arrs["B"], Br)
    _fill_slots(arrs["dt"], dtr)
    ring_start = torch.randint(0, L, (S,), generator=g, dtype=torch.int32).numpy()
    recur = None
    if spec.separate:  # drawn last, so the other values do not depend on the mode
        recur = arrs["recur"]
        h0r = torch.randn(S, H, P, N, generator=g, dtype=torch.float64) * h0_std
        _fill_slots(recur, _f16_bits(h0r.to(torch.float32)).view(np.uint8).reshape(S, -1))
    return CacheArrays(spec, arrs["state"], arrs["scale"], arrs["x"], arrs["B"], arrs["dt"],
                       ring_start.copy(), recur, gscale)


def make_params(spec: CacheSpec, seed: int):
    """Per-head parameters A, D, dt_bias (f32 [H])."""
    g = _gen(seed)
    H = spec.nheads
    A = -torch.exp(torch.rand(H, generator=g, dtype=torch.float64) * math.log(16.0))
    D = torch.randn(H, generator=g, dtype=torch.float64)
    dt_bias = -4.0 + 2.0 * torch.rand(H, generator=g, dtype=torch.float64)
    f = lambda t: t.to(torch.float32).numpy().copy()
    return f(A), f(D), f(dt_bias)


def make_step(spec: CacheSpec, batch: int, T: int, seed: int, pnat_max: int,
              varlen: bool = False, slots: Optional[np.ndarray] = None,
              n_padding: int = 0, pnat_fixed: Optional[int] = None, with_z: bool = False,
              dt_softplus: bool = True) -> StepInputs:
    """One decode step over `batch` entries.

    Active entries use unique random slots from [1, num_slots) (or `slots`);
    the first `n_padding` entries (after a seeded shuffle) are padding (slot 0).
    pnat ~ U{0..pnat_max} (or `pnat_fixed`); with `varlen`, T_b ~ U{1..T} and
    the inputs are packed along cu_seqlens.  `with_z` adds an output gate
    z ~ N(0, 1) in bf16 (drawn last, so the other values do not change);
    `dt_softplus` False draws dt so that dt + dt_bias follows the ring dt' law.
    """
    g = _gen(seed)
    H, G, P, N = spec.nheads, spec.ngroups, spec.headdim, spec.dstate
    if slots is None:
        perm = torch.randperm(spec.num_slots - 1, generator=g)[: batch - n_padding] + 1
        slots = np.concatenate([np.zeros(n_padding, np.int32), perm.numpy().astype(np.int32)])
        order = torch.randperm(batch, generator=g).numpy()
        slots = slots[order]
    slots = np.asarray(slots, np.int32)
    assert slots.shape == (batch,)
    if pnat_fixed is not None:
        pnat = np.full(batch, pnat_fixed, np.int32)
    else:
        pnat = torch.randint(0, pnat_max + 1, (batch,), generator=g, dtype=torch.int32).numpy()
    if varlen:
        Tb = torch.randint(1, T + 1, (batch,), generator=g, dtype=torch.int32).numpy()
        cu = np.zeros(batch + 1, np.int32)
        cu[1:] = np.cumsum(Tb)
        ntok = int(cu[-1])
    else:
        cu = None
        ntok = batch * T
    x = _bf16_bits(torch.randn(ntok, H, P, generator=g))
    B = _bf16_bits(torch.randn(ntok, G, N, generator=g))
    C = _bf16_bits(torch.randn(ntok, G, N, generator=g))
    dt = (torch.randn(ntok, H, generator=g, dtype=torch.float64) * 0.5).to(torch.float32).numpy()
    A, D, dt_bias = make_params(spec, seed + 7919)
    z = _bf16_bits(torch.randn(ntok, H, P, generator=g)) if with_z else None
    if not dt_softplus:
        # dt already processed by the caller: dt + dt_bias itself is the step
        # size, drawn with the ring dt' law (log-uniform on [0.004, 0.5])
        lo, hi = math.log(0.004), math.log(0.5)
        dtp = torch.exp(lo + (hi - lo) * torch.rand(ntok, H, generator=g, dtype=torch.float64))
        dt = (dtp - torch.from_numpy(dt_bias.astype(np.float64))[None, :]).to(torch.float32).numpy()
    return StepInputs(batch, T, slots, pnat.astype(np.int32), cu, x, B, C, dt, A, D, dt_bias, z,
                      dt_softplus)


# ---------------------------------------------------------------------------
# The five synthetic workloads (cache geometry, step shape, value laws above).
# ---------------------------------------------------------------------------

WORKLOADS = {
    # tiny reference: 2 active of 4 slots (slot 0 padding), fp32 state, T=1
    "tiny": dict(num_slots=4, nheads=8, ngroups=1, state_dtype="f32", batch=2, T=1,
                 pnat_max=8, out_dtype="f32"),
    # MTP decode: batch 64 of 128 slots, H64 G8, bf16 state, T=4 (1 + 3 drafts)
    "mtp": dict(num_slots=128, nheads=64, ngroups=8, state_dtype="bf16", batch=64, T=4,
                pnat_max=4, out_dtype="bf16"),
    # production mixed-pnat sweep: H128 G8, fp16 state, T=8 (1 + 7 drafts)
    "prod": dict(num_slots=None, nheads=128, ngroups=8, state_dtype="f16", batch=256, T=8,
                 pnat_max=8, out_dtype="bf16"),
    # quantised checkpoint: batch 256, fp8 e4m3 + row scales, T=4, flush every step
    "fp8": dict(num_slots=None, nheads=128, ngroups=8, state_dtype="fp8", batch=256, T=4,
                pnat_max=0, out_dtype="bf16", flush_k=(1, 4)),
    # large batch: 1024 active of 2048 slots, bf16 state, varlen T_b ~ U{1..8}, 256 B slot pad
    "large": dict(num_slots=2048, nheads=128, ngroups=8, state_dtype="bf16", batch=1024, T=8,
                  pnat_max=8, out_dtype="bf16", varlen=True, slot_pad=256),
}


def flush_counts(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """k ~ U{lo..hi} per entry (int32)."""
    g = _gen(seed)
    return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int32).numpy()
