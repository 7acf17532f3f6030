"""Python front end of the CPU oracle (oracle/ssu_oracle.c).  TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module; the product path never imports it.  It loads (building it with gcc if
it is missing) the plain fp64 C implementation and passes numpy buffers to it.
The cache and step objects are the ones `synth` generates (attribute access
only; nothing else is shared with the GPU library).

Functions:
  replay_step(cache, step)              -> (out fp64 [tokens, H, P], status)
  flush(cache, slot_idx, num_fold, A)   -> status
  init_state(cache, states, slot_idx, states_stride=None)
  encoders / decoders / softplus on arrays, for the pins.
The cache passed in is modified in place (ring appends, flushed checkpoints,
ring_start), exactly as the library modifies device memory.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssu_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssu_oracle.so")
_lock = threading.Lock()
_lib = None

_DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2, "fp8": 3, "f64": 4, "nvfp4": 5}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into oracle/libssu_oracle.so."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _OrCache(ctypes.Structure):
    _fields_ = [
        ("num_slots", ctypes.c_int), ("nheads", ctypes.c_int), ("ngroups", ctypes.c_int),
        ("headdim", ctypes.c_int), ("dstate", ctypes.c_int), ("ring_len", ctypes.c_int),
        ("state_dtype", ctypes.c_int), ("state_layout", ctypes.c_int),
        ("state", ctypes.c_void_p), ("state_stride", ctypes.c_int64),
        ("scale", ctypes.c_void_p), ("scale_stride", ctypes.c_int64),
        ("x_cache", ctypes.c_void_p), ("x_stride", ctypes.c_int64),
        ("B_cache", ctypes.c_void_p), ("B_stride", ctypes.c_int64),
        ("dt_cache", ctypes.c_void_p), ("dt_stride", ctypes.c_int64),
        ("ring_start", ctypes.c_void_p),
        ("recur", ctypes.c_void_p), ("recur_stride", ctypes.c_int64),
        ("gscale", ctypes.c_void_p), ("gscale_stride", ctypes.c_int64),
    ]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            L = ctypes.CDLL(build())
            P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
            L.or_replay_step.restype = I
            L.or_replay_step.argtypes = [ctypes.POINTER(_OrCache), I, I, P, P, P, P, P, P, P,
                                         P, P, P, P, I, P]
            L.or_flush.restype = I
            L.or_flush.argtypes = [ctypes.POINTER(_OrCache), I, P, P, P, ctypes.c_uint64]
            L.or_init_state.restype = None
            L.or_init_state.argtypes = [ctypes.POINTER(_OrCache), P, I64, P, I, ctypes.c_uint64]
            L.or_philox4x32.restype = None
            L.or_philox4x32.argtypes = [P, P, I, P]
            L.or_sr_f16_array.restype = None
            L.or_sr_f16_array.argtypes = [P, P, P, I64]
            L.or_sr_bits_array.restype = None
            L.or_sr_bits_array.argtypes = [ctypes.c_uint64, I, I, P, I64]
            L.or_decode_head.restype = None
            L.or_decode_head.argtypes = [ctypes.POINTER(_OrCache), I, I, P]
            L.or_encode_slot_nvfp4.restype = None
            L.or_encode_slot_nvfp4.argtypes = [ctypes.POINTER(_OrCache), I, P]
            for name in ("or_enc_bf16_array", "or_enc_f16_array", "or_enc_e4m3_array",
                         "or_bf16_value_array", "or_f16_value_array", "or_e4m3_value_array",
                         "or_e2m1_value_array", "or_enc_e2m1_array", "or_softplus_array"):
                f = getattr(L, name)
                f.restype = None
                f.argtypes = [P, P, I64]
            L.or_set_threads.restype = None
            L.or_set_threads.argtypes = [I]
            L.or_max_threads.restype = I
            L.or_max_threads.argtypes = []
            L.or_init_tables()
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _as_orcache(cache) -> _OrCache:
    s = cache.spec
    for a in (cache.state, cache.scale, cache.x_cache, cache.B_cache, cache.dt_cache,
              cache.ring_start):
        assert a.flags["C_CONTIGUOUS"]
    assert cache.ring_start.dtype == np.int32
    recur = getattr(cache, "recur", None)
    assert recur is None or recur.flags["C_CONTIGUOUS"]
    gscale = getattr(cache, "gscale", None)
    assert gscale is None or gscale.flags["C_CONTIGUOUS"]
    return _OrCache(
        s.num_slots, s.nheads, s.ngroups, s.headdim, s.dstate, s.ring_len,
        _DTYPE_CODE[s.state_dtype], {"rowmajor": 0, "tiled": 1}[s.state_layout],
        cache.state.ctypes.data, cache.state.shape[1],
        cache.scale.ctypes.data, cache.scale.shape[1],
        cache.x_cache.ctypes.data, cache.x_cache.shape[1],
        cache.B_cache.ctypes.data, cache.B_cache.shape[1],
        cache.dt_cache.ctypes.data, cache.dt_cache.shape[1],
        cache.ring_start.ctypes.data,
        None if recur is None else recur.ctypes.data, 0 if recur is None else recur.shape[1],
        None if gscale is None else gscale.ctypes.data, 0 if gscale is None else gscale.shape[1])


_STATUS_BAD_FOLD = 2


def replay_step(cache, step, num_fold=None, seed=0):
    """Replay step (see or_replay_step).  Returns (out fp64 [tokens, H, P], status).

    The step's optional `z` (bf16 bits like x) gates the output with
    z * sigmoid(z); `dt_softplus` False makes dt' = dt + dt_bias.

    With num_fold ([batch] ints) the step is the fused flush-in-step: for each
    entry the step would process (valid slot, 0 <= pnat, pnat + T_b <= L, a
    valid ring_start and T_b within max_seqlen) and k = num_fold[b] in
    [0, pnat], the first k live tokens are flushed into the checkpoint and the
    step then runs with pnat - k live tokens from the new ring start; an entry
    with k outside [0, pnat] is skipped like padding (zero output rows, cache
    untouched) and reported with status bit 2.  This is by definition the
    composition of flush (with `seed`) and replay_step below.
    """
    if num_fold is not None:
        return _fused_step(cache, step, np.asarray(num_fold, np.int32), seed)
    s = cache.spec
    oc = _as_orcache(cache)
    ntok = step.tokens
    out = np.full((ntok, s.nheads, s.headdim), np.nan, np.float64)
    x = _c(step.x, np.uint16)
    B = _c(step.B, np.uint16)
    C = _c(step.C, np.uint16)
    dt = _c(step.dt, np.float32)
    A = _c(step.A, np.float32)
    D = _c(step.D, np.float32)
    db = _c(step.dt_bias, np.float32)
    slots = _c(step.slot_idx, np.int32)
    pnat = _c(step.pnat, np.int32)
    cu = None if step.cu_seqlens is None else _c(step.cu_seqlens, np.int32)
    z = getattr(step, "z", None)
    z = None if z is None else _c(z, np.uint16)
    assert x.shape == (ntok, s.nheads, s.headdim) and B.shape == (ntok, s.ngroups, s.dstate)
    assert z is None or z.shape == x.shape
    st = lib().or_replay_step(ctypes.byref(oc), step.batch, step.T, _ptr(cu), _ptr(slots),
                              _ptr(pnat), _ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A),
                              _ptr(D), _ptr(db), _ptr(z), int(getattr(step, "dt_softplus", True)),
                              out.ctypes.data)
    return out, st


def _fused_step(cache, step, k, seed):
    s = cache.spec
    assert k.shape == (step.batch,)
    if step.cu_seqlens is not None:
        tb = np.diff(np.asarray(step.cu_seqlens, np.int64))
    else:
        tb = np.full(step.batch, step.T, np.int64)
    slots = np.asarray(step.slot_idx, np.int32).copy()
    pnat = np.asarray(step.pnat, np.int32).copy()
    status = 0
    fold_slots, fold_k = [], []
    for b in range(step.batch):
        sl, p = int(slots[b]), int(pnat[b])
        if not (0 <= tb[b] <= step.T) or not (0 < sl < s.num_slots):
            continue
        if p < 0 or p + tb[b] > s.ring_len:
            continue
        if not (0 <= int(cache.ring_start[sl]) < s.ring_len):
            continue
        kb = int(k[b])
        if kb < 0 or kb > p:
            status |= _STATUS_BAD_FOLD
            slots[b] = 0  # skipped like a padding entry
            continue
        if kb > 0:
            fold_slots.append(sl)
            fold_k.append(kb)
            pnat[b] = p - kb
    if fold_slots:
        st = flush(cache, np.array(fold_slots, np.int32), np.array(fold_k, np.int32), step.A, seed)
        assert st == 0
    sub = _replace(step, slot_idx=slots, pnat=pnat)
    out, st = replay_step(cache, sub)
    return out, st | status


def _replace(step, **kw):
    import dataclasses
    return dataclasses.replace(step, **kw)


def flush(cache, slot_idx, num_fold, A, seed=0):
    """Fold the first k live ring tokens into each listed slot's checkpoint
    (with a recurrence checkpoint: fold from it, write it back with
    stochastic rounding drawn from `seed`, and re-encode the read one)."""
    oc = _as_orcache(cache)
    slots = _c(slot_idx, np.int32)
    k = _c(num_fold, np.int32)
    A = _c(A, np.float32)
    assert slots.shape == k.shape
    return lib().or_flush(ctypes.byref(oc), slots.shape[0], _ptr(slots), _ptr(k), _ptr(A),
                          ctypes.c_uint64(int(seed)))


def init_state(cache, states, slot_idx, states_stride=None, seed=0):
    """Encode fp32 states [n, H, P, N] into the listed slots and clear their rings."""
    s = cache.spec
    oc = _as_orcache(cache)
    states = np.asarray(states, np.float32)
    slots = _c(slot_idx, np.int32)
    if states_stride is None:
        states = np.ascontiguousarray(states)
        states_stride = s.nheads * s.headdim * s.dstate
    lib().or_init_state(ctypes.byref(oc), states.ctypes.data, int(states_stride), _ptr(slots),
                        slots.shape[0], ctypes.c_uint64(int(seed)))


def set_threads(n: int) -> None:
    """Number of OpenMP threads the oracle's loops use from now on."""
    lib().or_set_threads(int(n))


def max_threads() -> int:
    return int(lib().or_max_threads())


def philox4x32(ctr, key, rounds=10):
    """Philox4x32 with the given round count: four 32-bit counter words and
    two key words in, four words out."""
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    assert c.shape == (4,) and k.shape == (2,)
    out = np.empty(4, np.uint32)
    lib().or_philox4x32(c.ctypes.data, k.ctypes.data, int(rounds), out.ctypes.data)
    return out


def sr_f16(v, u):
    """Stochastic rounding of fp32 values to fp16 bits with 7-bit randoms u."""
    v = np.ascontiguousarray(v, np.float32)
    u = np.ascontiguousarray(u, np.uint8)
    assert v.shape == u.shape
    out = np.empty(v.shape, np.uint16)
    lib().or_sr_f16_array(v.ctypes.data, u.ctypes.data, out.ctypes.data, v.size)
    return out


def sr_bits(seed, slot, head, n):
    """The 7-bit randoms of values 0..n-1 of (slot, head) for `seed`."""
    out = np.empty(n, np.uint8)
    lib().or_sr_bits_array(ctypes.c_uint64(int(seed)), int(slot), int(head), out.ctypes.data, n)
    return out


def encode_slot_nvfp4(cache, slot, values):
    """Encode fp32 [H, P, N] values into one slot of an NVFP4 checkpoint (one
    second-level scale over every head of the slot)."""
    s = cache.spec
    v = np.ascontiguousarray(values, np.float32)
    assert v.shape == (s.nheads, s.headdim, s.dstate)
    oc = _as_orcache(cache)
    lib().or_encode_slot_nvfp4(ctypes.byref(oc), int(slot), v.ctypes.data)


def e2m1_value(b):
    return _arr("or_e2m1_value_array", b, np.uint8, np.float64)


def enc_e2m1(v):
    return _arr("or_enc_e2m1_array", v, np.float64, np.uint8)


def decode_recur(cache, slot):
    """fp64 [H, P, N] value of one slot's FP16 recurrence checkpoint."""
    return f16_value(cache.recur_logical(slot))


def _arr(fn, a, in_dtype, out_dtype):
    a = np.ascontiguousarray(a, dtype=in_dtype)
    out = np.empty(a.shape, out_dtype)
    getattr(lib(), fn)(a.ctypes.data, out.ctypes.data, a.size)
    return out


def enc_bf16(v):
    return _arr("or_enc_bf16_array", v, np.float64, np.uint16)


def enc_f16(v):
    return _arr("or_enc_f16_array", v, np.float64, np.uint16)


def enc_e4m3(v):
    return _arr("or_enc_e4m3_array", v, np.float64, np.uint8)


def bf16_value(b):
    return _arr("or_bf16_value_array", b, np.uint16, np.float64)


def f16_value(b):
    return _arr("or_f16_value_array", b, np.uint16, np.float64)


def e4m3_value(b):
    return _arr("or_e4m3_value_array", b, np.uint8, np.float64)


def softplus(v):
    return _arr("or_softplus_array", v, np.float64, np.float64)


def decode_state(cache, slot):
    """fp64 [H, P, N] value of one slot's checkpoint (decode rule of the oracle)."""
    s = cache.spec
    if s.state_dtype == "nvfp4":
        oc = _as_orcache(cache)
        out = np.empty((s.nheads, s.headdim, s.dstate), np.float64)
        for h in range(s.nheads):
            lib().or_decode_head(ctypes.byref(oc), int(slot), h, out[h].ctypes.data)
        return out
    raw = cache.state_logical(slot)
    if s.state_dtype in ("f32", "f64"):
        return raw.astype(np.float64)
    if s.state_dtype == "bf16":
        return bf16_value(raw)
    if s.state_dtype == "f16":
        return f16_value(raw)
    return e4m3_value(raw) * cache.scale_view(slot).astype(np.float64)[:, :, None]
