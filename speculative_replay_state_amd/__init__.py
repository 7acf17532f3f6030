"""Python binding of libssu (include/ssu.h): the checkpointing selective state
update (ReplaySSM / MTP-replay SSU) on AMD MI355X.

This module only marshals arguments: it builds the C descriptors from device
tensors and calls the library.  Every step of the computation runs in the
library's HIP kernels.  Importing fails loudly when libssu.so has not been
built (python speculative_replay_state_amd/build.py); there is no fallback.

Names follow the C ABI: ssu_init_state, ssu_replay_step, ssu_flush,
ssu_workspace_size, ssu_resolve_algo, ssu_last_error, plus DeviceCache (the
device tensors of one cache, in the layout of ssu_cache) and replay_step /
flush / init_state helpers that take torch tensors.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssu.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libssu.so is not built at %s; run `python speculative_replay_state_amd/build.py` "
        "(needs ROCm hipcc)" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

# ssu_dtype / ssu_algo / return codes / status bits (include/ssu.h)
SSU_F32, SSU_BF16, SSU_F16, SSU_FP8_E4M3, SSU_NVFP4 = 0, 1, 2, 3, 4
SSU_ALGO_AUTO, SSU_ALGO_MONOLITH, SSU_ALGO_SPLIT = 0, 1, 2
SSU_OK, SSU_ERR_INVALID, SSU_ERR_UNSUPPORTED, SSU_ERR_HIP, SSU_ERR_WORKSPACE = 0, -1, -2, -3, -4
SSU_STATUS_BAD_PNAT, SSU_STATUS_BAD_FOLD, SSU_STATUS_BAD_SEQLEN, SSU_STATUS_BAD_RING = 1, 2, 4, 8

DTYPE_CODES = {"f32": SSU_F32, "bf16": SSU_BF16, "f16": SSU_F16, "fp8": SSU_FP8_E4M3, "nvfp4": SSU_NVFP4}
ALGO_CODES = {"auto": SSU_ALGO_AUTO, "monolith": SSU_ALGO_MONOLITH, "split": SSU_ALGO_SPLIT}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


class SsuCache(ctypes.Structure):
    _fields_ = [
        ("num_slots", _I32), ("nheads", _I32), ("ngroups", _I32), ("headdim", _I32),
        ("dstate", _I32), ("ring_len", _I32),
        ("state_dtype", ctypes.c_int), ("io_dtype", ctypes.c_int),
        ("state", _P), ("state_slot_stride", _I64),
        ("state_scale", _P), ("scale_slot_stride", _I64),
        ("x_cache", _P), ("x_slot_stride", _I64),
        ("B_cache", _P), ("B_slot_stride", _I64),
        ("dt_cache", _P), ("dt_slot_stride", _I64),
        ("ring_start", _P), ("status", _P),
        ("recur_state", _P), ("recur_slot_stride", _I64),
        ("state_gscale", _P), ("gscale_slot_stride", _I64),
    ]


class SsuStep(ctypes.Structure):
    _fields_ = [
        ("batch", _I32), ("max_seqlen", _I32),
        ("slot_idx", _P), ("prev_num_accepted", _P), ("cu_seqlens", _P),
        ("x", _P), ("B", _P), ("C", _P), ("dt", _P),
        ("A", _P), ("D", _P), ("dt_bias", _P),
        ("out", _P), ("out_dtype", ctypes.c_int),
        ("workspace", _P), ("workspace_bytes", ctypes.c_size_t), ("algo", ctypes.c_int),
        ("num_fold", _P), ("z", _P), ("no_dt_softplus", _I32), ("sr_seed", ctypes.c_uint64),
    ]


_lib.ssu_workspace_size.restype = ctypes.c_size_t
_lib.ssu_workspace_size.argtypes = [ctypes.POINTER(SsuCache), _I32, _I32]
_lib.ssu_init_state.restype = ctypes.c_int
_lib.ssu_init_state.argtypes = [ctypes.POINTER(SsuCache), _P, _I64, _P, _I32, ctypes.c_uint64, _P]
_lib.ssu_replay_step.restype = ctypes.c_int
_lib.ssu_replay_step.argtypes = [ctypes.POINTER(SsuCache), ctypes.POINTER(SsuStep), _P]
_lib.ssu_replay_step_noalloc.restype = ctypes.c_int
_lib.ssu_replay_step_noalloc.argtypes = [ctypes.POINTER(SsuCache), ctypes.POINTER(SsuStep), _P]
_lib.ssu_flush.restype = ctypes.c_int
_lib.ssu_flush.argtypes = [ctypes.POINTER(SsuCache), _P, _P, _P, _I32, ctypes.c_uint64, _P]
_lib.ssu_resolve_algo.restype = ctypes.c_int
_lib.ssu_resolve_algo.argtypes = [ctypes.POINTER(SsuCache), ctypes.POINTER(SsuStep)]
_lib.ssu_get_split_threshold.restype = _I64
_lib.ssu_get_split_threshold.argtypes = []
_lib.ssu_set_split_threshold.restype = _I64
_lib.ssu_set_split_threshold.argtypes = [_I64]
_lib.ssu_last_error.restype = ctypes.c_char_p
_lib.ssu_last_error.argtypes = []

EXPORTED = ("ssu_workspace_size", "ssu_init_state", "ssu_replay_step", "ssu_replay_step_noalloc", "ssu_flush",
            "ssu_resolve_algo", "ssu_get_split_threshold", "ssu_set_split_threshold",
            "ssu_last_error")
SSU_NOALLOC_SCRATCH_BYTES = 16 << 20
SSU_MAX_PAIRS = (1 << 24) - 1


class SsuError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("libssu error %d: %s" % (code, message))
        self.code = code


def ssu_last_error() -> str:
    return (_lib.ssu_last_error() or b"").decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise SsuError(rc, ssu_last_error())
    return rc


# ---------------------------------------------------------------------------
# raw C entry points (descriptor structs in, return code out)
# ---------------------------------------------------------------------------

def ssu_workspace_size(cache: SsuCache, batch: int, max_seqlen: int) -> int:
    return int(_lib.ssu_workspace_size(ctypes.byref(cache), batch, max_seqlen))


def ssu_init_state(cache: SsuCache, states: int, states_batch_stride: int, slot_idx: int, n: int,
                   sr_seed: int = 0, stream: int = 0) -> int:
    return _lib.ssu_init_state(ctypes.byref(cache), states, states_batch_stride, slot_idx, n, sr_seed,
                               stream)


def ssu_replay_step(cache: SsuCache, step: SsuStep, stream: int = 0) -> int:
    return _lib.ssu_replay_step(ctypes.byref(cache), ctypes.byref(step), stream)


def ssu_replay_step_noalloc(cache: SsuCache, step: SsuStep, stream: int = 0) -> int:
    return _lib.ssu_replay_step_noalloc(ctypes.byref(cache), ctypes.byref(step), stream)


def ssu_flush(cache: SsuCache, slot_idx: int, num_fold: int, A: int, n: int, sr_seed: int = 0,
              stream: int = 0) -> int:
    return _lib.ssu_flush(ctypes.byref(cache), slot_idx, num_fold, A, n, sr_seed, stream)


def ssu_resolve_algo(cache: SsuCache, step: SsuStep) -> int:
    return _lib.ssu_resolve_algo(ctypes.byref(cache), ctypes.byref(step))


def ssu_get_split_threshold() -> int:
    return int(_lib.ssu_get_split_threshold())


def ssu_set_split_threshold(work_units: int) -> int:
    return int(_lib.ssu_set_split_threshold(work_units))


# ---------------------------------------------------------------------------
# torch-tensor front end (argument marshalling only)
# ---------------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _on_device(t, name: str):
    """A tensor the kernels may address: on the GPU (a host pointer handed to
    a kernel faults the device)."""
    if t is not None and not getattr(t, "is_cuda", False):
        raise ValueError("%s must be a device tensor (got one on %s)" % (name, getattr(t, "device", "?")))


def _packed(t, name: str, nbytes: Optional[int] = None):
    """A device tensor whose bytes are packed (C-contiguous) and, when
    `nbytes` is given, at least that many."""
    if t is None:
        return
    _on_device(t, name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    have = t.numel() * t.element_size()
    if nbytes is not None and have < nbytes:
        raise ValueError("%s holds %d bytes; the step addresses %d" % (name, have, nbytes))


def _slot_pages(t, name: str, num_slots: int) -> int:
    """Byte stride between the slot pages of a per-slot cache tensor
    [num_slots, ...] whose pages are each packed (the rows may be padded)."""
    _on_device(t, name)
    if t.dim() < 2 or t.shape[0] != num_slots:
        raise ValueError("%s must be [num_slots=%d, ...] (got shape %s)" % (name, num_slots, tuple(t.shape)))
    if not t[0].is_contiguous():
        raise ValueError("%s: each slot page must be contiguous" % name)
    return t.stride(0) * t.element_size()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclasses.dataclass
class DeviceCache:
    """Device tensors of one cache in the ssu_cache layout.

    Every per-slot tensor is a uint8 tensor [num_slots, slot_stride_bytes]
    (the packed slot layout of include/ssu.h, plus optional padding);
    ring_start is int32 [num_slots]; status is an optional int32 [1].
    """
    num_slots: int
    nheads: int
    ngroups: int
    ring_len: int
    state_dtype: str
    state: object
    scale: object
    x_cache: object
    B_cache: object
    dt_cache: object
    ring_start: object
    status: object = None
    headdim: int = 64
    dstate: int = 128
    recur: object = None  # FP16 recurrence checkpoint (separate checkpoints) or None
    gscale: object = None  # nvfp4: uint8 [num_slots, stride]: f32 slot scale, then the head maxima

    def desc(self) -> SsuCache:
        """The C descriptor.  Raises ValueError for a tensor the kernels could
        not address as the layout says: on the host, not num_slots pages, a
        page that is not contiguous, or ring_start / status too small."""
        scaled = self.state_dtype in ("fp8", "nvfp4")
        nvfp4 = self.state_dtype == "nvfp4"
        n = self.num_slots

        def pages(t, name):
            return _slot_pages(t, name, n)

        _packed(self.ring_start, "ring_start", 4 * n)
        _packed(self.status, "status", 4)
        return SsuCache(
            n, self.nheads, self.ngroups, self.headdim, self.dstate, self.ring_len,
            DTYPE_CODES[self.state_dtype], SSU_BF16,
            _ptr(self.state), pages(self.state, "state"),
            _ptr(self.scale) if scaled else None, pages(self.scale, "scale") if scaled else 0,
            _ptr(self.x_cache), pages(self.x_cache, "x_cache"),
            _ptr(self.B_cache), pages(self.B_cache, "B_cache"),
            _ptr(self.dt_cache), pages(self.dt_cache, "dt_cache"),
            _ptr(self.ring_start), _ptr(self.status),
            _ptr(self.recur), 0 if self.recur is None else pages(self.recur, "recur"),
            _ptr(self.gscale) if nvfp4 else None, pages(self.gscale, "gscale") if nvfp4 else 0)


def make_step_desc(batch, max_seqlen, slot_idx, pnat, cu_seqlens, x, B, C, dt, A, D, dt_bias, out,
                   out_dtype="bf16", workspace=None, algo="auto", num_fold=None, z=None,
                   dt_softplus=True, sr_seed=0) -> SsuStep:
    """The ssu_step descriptor of one step, from device tensors.

    slot_idx, pnat (live ring tokens ahead of the new ones), num_fold: int32
    [batch]; cu_seqlens: int32 [batch + 1] or None (every entry then has
    max_seqlen tokens, token t of entry b in row b * max_seqlen + t); x, z:
    bf16 [rows, H, 64]; B, C: bf16 [rows, G, 128]; dt: f32 [rows, H]; A, D,
    dt_bias: f32 [H]; out: [rows, H, 64] of out_dtype ("bf16" or "f32").
    algo: "auto", "monolith" or "split" (split needs `workspace` of
    workspace_size(cache, batch, max_seqlen) bytes).  num_fold folds the
    first k live tokens of each entry before its readout (fused flush-in-
    step); z gates the output; dt_softplus=False takes dt' = dt + dt_bias;
    sr_seed keys the stochastic rounding of a fused fold into an FP16
    recurrence checkpoint (pass a new one on every call)."""
    desc = SsuStep(
        batch, max_seqlen, _ptr(slot_idx), _ptr(pnat), _ptr(cu_seqlens),
        _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(D), _ptr(dt_bias),
        _ptr(out), SSU_F32 if out_dtype == "f32" else SSU_BF16,
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        ALGO_CODES[algo], _ptr(num_fold), _ptr(z), 0 if dt_softplus else 1, int(sr_seed))
    # The descriptor holds raw device pointers: it keeps the tensors they point
    # into alive, so that memory a kernel (or a captured graph) writes is never
    # handed to another tensor while the descriptor is in use.
    desc._tensors = dict(slot_idx=slot_idx, prev_num_accepted=pnat, cu_seqlens=cu_seqlens, x=x, B=B, C=C, dt=dt,
                         A=A, D=D, dt_bias=dt_bias, out=out, workspace=workspace, num_fold=num_fold, z=z)
    return desc


def check_step_tensors(cache: DeviceCache, step: SsuStep):
    """The tensors of a step descriptor made by make_step_desc are device
    tensors, packed, and (with a fixed T per entry) as large as the layouts of
    include/ssu.h make the step address; the library checks the rest.  With
    cu_seqlens the row count lives on the device, so only the per-entry and
    per-head arrays are sized here.  Raises ValueError."""
    t = getattr(step, "_tensors", None)
    if t is None or step.batch <= 0:
        return
    H, G, b = cache.nheads, cache.ngroups, step.batch
    rows = None if t["cu_seqlens"] is not None else b * step.max_seqlen
    out_bytes = 4 if step.out_dtype == SSU_F32 else 2
    sizes = dict(slot_idx=4 * b, prev_num_accepted=4 * b, cu_seqlens=4 * (b + 1), num_fold=4 * b,
                 A=4 * H, D=4 * H, dt_bias=4 * H, workspace=None)
    if rows is not None:
        sizes.update(x=rows * H * 64 * 2, B=rows * G * 128 * 2, C=rows * G * 128 * 2, dt=rows * H * 4,
                     out=rows * H * 64 * out_bytes, z=rows * H * 64 * 2)
    for name, tensor in t.items():
        _packed(tensor, name, sizes.get(name))


def workspace_size(cache: DeviceCache, batch: int, max_seqlen: int) -> int:
    """Bytes of scratch a SPLIT step of (batch, max_seqlen) needs (0 when the
    cache or the sizes are invalid)."""
    return ssu_workspace_size(cache.desc(), batch, max_seqlen)


def init_state(cache: DeviceCache, states, slot_idx, states_batch_stride=None, stream=None, sr_seed=0):
    """ssu_init_state with torch tensors (states f32 [n, H, 64, 128] on device)."""
    n = slot_idx.numel()
    _on_device(states, "states")
    _packed(slot_idx, "slot_idx")
    if states_batch_stride is None:
        states_batch_stride = states.stride(0) if n else 0
    _check(ssu_init_state(cache.desc(), _ptr(states), states_batch_stride, _ptr(slot_idx), n,
                          int(sr_seed), _stream(stream)))


def replay_step(cache: DeviceCache, step: SsuStep, stream=None):
    """ssu_replay_step: read out the step's tokens into step's `out` and append
    them to the rings (with num_fold: fold first, and advance ring_start).
    Raises ValueError for tensors the kernels could not address, SsuError for
    a code the library returns."""
    check_step_tensors(cache, step)
    _check(ssu_replay_step(cache.desc(), step, _stream(stream)))


def replay_step_noalloc(cache: DeviceCache, step: SsuStep, stream=None):
    """ssu_replay_step_noalloc: replay_step with the SPLIT scratch taken from
    the library's own device array (step's workspace is ignored)."""
    check_step_tensors(cache, step)
    _check(ssu_replay_step_noalloc(cache.desc(), step, _stream(stream)))


def flush(cache: DeviceCache, slot_idx, num_fold, A, stream=None, sr_seed=0):
    """ssu_flush: fold the first num_fold[j] live ring tokens of slot
    slot_idx[j] into its checkpoint, re-encode it and advance ring_start
    (slot_idx, num_fold: int32 [n]; A: f32 [H], the steps' A)."""
    n = slot_idx.numel()
    _packed(slot_idx, "slot_idx")
    _packed(num_fold, "num_fold", 4 * n)
    _packed(A, "A", 4 * cache.nheads)
    _check(ssu_flush(cache.desc(), _ptr(slot_idx), _ptr(num_fold), _ptr(A), slot_idx.numel(), int(sr_seed),
                     _stream(stream)))
