"""The C ABI without a GPU: libssu.so loads, exports every function that
include/ssu.h declares, and rejects bad arguments on the host (returning the
documented error code and message) before any kernel launch.  The pointers
below are never dereferenced: every call here fails validation first.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssu.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return sorted(set(re.findall(r"\b(ssu_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def ssu():
    import speculative_replay_state_amd as m
    return m


def test_exports_every_declared_symbol(ssu):
    names = _declared_functions()
    assert {"ssu_init_state", "ssu_replay_step", "ssu_flush", "ssu_workspace_size"} <= set(names)
    lib = ctypes.CDLL(ssu.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ssu.EXPORTED)


FAKE = 0x10000  # 16-byte aligned, never dereferenced


def _cache(ssu, **kw):
    d = dict(num_slots=8, nheads=16, ngroups=2, headdim=64, dstate=128, ring_len=16,
             state_dtype=ssu.SSU_BF16, io_dtype=ssu.SSU_BF16,
             state=FAKE, state_slot_stride=16 * 64 * 128 * 2,
             state_scale=FAKE, scale_slot_stride=16 * 64 * 4,
             x_cache=FAKE, x_slot_stride=16 * 16 * 64 * 2,
             B_cache=FAKE, B_slot_stride=2 * 16 * 128 * 2,
             dt_cache=FAKE, dt_slot_stride=16 * 16 * 4,
             ring_start=FAKE, status=None)
    d.update(kw)
    c = ssu.SsuCache()
    for k, v in d.items():
        setattr(c, k, v)
    return c


def _step(ssu, **kw):
    d = dict(batch=4, max_seqlen=4, slot_idx=FAKE, prev_num_accepted=FAKE, cu_seqlens=None,
             x=FAKE, B=FAKE, C=FAKE, dt=FAKE, A=FAKE, D=FAKE, dt_bias=FAKE, out=FAKE,
             out_dtype=ssu.SSU_BF16, workspace=None, workspace_bytes=0, algo=ssu.SSU_ALGO_SPLIT)
    d.update(kw)
    s = ssu.SsuStep()
    for k, v in d.items():
        setattr(s, k, v)
    return s


CACHE_ERRORS = [
    (dict(headdim=32), -2, "headdim"),
    (dict(dstate=64), -2, "dstate"),
    (dict(nheads=15), -1, "multiple"),
    (dict(ring_len=33), -2, "ring_len"),
    (dict(ring_len=0), -2, "ring_len"),
    (dict(num_slots=0), -1, "positive"),
    (dict(state=None), -1, "NULL"),
    (dict(ring_start=None), -1, "NULL"),
    (dict(state=FAKE + 8), -1, "aligned"),
    (dict(state_dtype=7), -1, "state_dtype"),
    (dict(io_dtype=0), -2, "io_dtype"),
    (dict(state_dtype=3, state_scale=None), -1, "state_scale"),
    (dict(state_slot_stride=100), -1, "stride"),
    (dict(x_slot_stride=16 * 16 * 64 * 2 + 8), -1, "multiple of 16"),
]


@pytest.mark.parametrize("kw,code,msg", CACHE_ERRORS)
def test_cache_validation(ssu, kw, code, msg):
    c = _cache(ssu, **kw)
    assert ssu.ssu_replay_step(c, _step(ssu)) == code
    assert msg in ssu.ssu_last_error()
    assert ssu.ssu_flush(c, FAKE, FAKE, FAKE, 3, 1) == code
    assert ssu.ssu_init_state(c, FAKE, 0, FAKE, 3, 1) == code
    assert ssu.ssu_workspace_size(c, 4, 4) == 0


STEP_ERRORS = [
    (dict(max_seqlen=0), -1, "max_seqlen"),
    (dict(max_seqlen=17), -1, "exceeds"),
    (dict(batch=-1), -1, "batch"),
    (dict(x=None), -1, "NULL"),
    (dict(out=None), -1, "NULL"),
    (dict(out=FAKE + 4), -1, "aligned"),
    (dict(dt=FAKE + 2), -1, "aligned"),
    (dict(out_dtype=2), -2, "out_dtype"),
    (dict(algo=9), -1, "algo"),
    (dict(workspace=None), -4, "workspace"),
    (dict(workspace=FAKE, workspace_bytes=16), -4, "workspace"),
    (dict(num_fold=FAKE), -2, "monolith only"),
    (dict(num_fold=FAKE + 2, algo=0), -1, "num_fold"),
    (dict(z=FAKE + 8), -1, "z must be 16-byte aligned"),
    (dict(batch=(1 << 24) // 16), -2, "SSU_MAX_PAIRS"),  # 16 heads: one pair past the bound
]


@pytest.mark.parametrize("kw,code,msg", STEP_ERRORS)
def test_step_validation(ssu, kw, code, msg):
    assert ssu.ssu_replay_step(_cache(ssu), _step(ssu, **kw)) == code
    assert msg in ssu.ssu_last_error()


def test_tokens_above_16_unsupported_when_ring_allows(ssu):
    c = _cache(ssu, ring_len=32, x_slot_stride=16 * 32 * 64 * 2, B_slot_stride=2 * 32 * 128 * 2,
               dt_slot_stride=16 * 32 * 4)
    assert ssu.ssu_replay_step(c, _step(ssu, max_seqlen=17)) == -2


def test_workspace_size_and_algo_resolution(ssu):
    c = _cache(ssu)
    assert ssu.ssu_workspace_size(c, 4, 4) == 4 * 2 * 4 * 32 * 4
    assert ssu.ssu_workspace_size(c, 0, 4) == 0
    old = ssu.ssu_set_split_threshold(64)
    try:
        assert ssu.ssu_get_split_threshold() == 64
        s = _step(ssu, algo=ssu.SSU_ALGO_AUTO, batch=4)  # 4 x 16 heads = 64 units
        assert ssu.ssu_resolve_algo(c, s) == ssu.SSU_ALGO_SPLIT
        s = _step(ssu, algo=ssu.SSU_ALGO_AUTO, batch=3)
        assert ssu.ssu_resolve_algo(c, s) == ssu.SSU_ALGO_MONOLITH
        s = _step(ssu, algo=ssu.SSU_ALGO_MONOLITH, batch=400)
        assert ssu.ssu_resolve_algo(c, s) == ssu.SSU_ALGO_MONOLITH
        s = _step(ssu, algo=ssu.SSU_ALGO_AUTO, batch=400, num_fold=FAKE)  # fused: monolith
        assert ssu.ssu_resolve_algo(c, s) == ssu.SSU_ALGO_MONOLITH
    finally:
        ssu.ssu_set_split_threshold(old)


def test_auto_defaults_to_monolith(ssu):
    c = _cache(ssu)
    s = _step(ssu, algo=ssu.SSU_ALGO_AUTO, batch=100000)
    assert ssu.ssu_resolve_algo(c, s) == ssu.SSU_ALGO_MONOLITH


def test_pairs_per_call_bound(ssu):
    c = _cache(ssu)  # 16 heads
    n_max = ssu.SSU_MAX_PAIRS // 16
    assert ssu.ssu_resolve_algo(c, _step(ssu, batch=n_max)) == ssu.SSU_ALGO_SPLIT
    assert ssu.ssu_flush(c, FAKE, FAKE, FAKE, n_max + 1) == -2
    assert "SSU_MAX_PAIRS" in ssu.ssu_last_error()
    assert ssu.ssu_init_state(c, FAKE, 0, FAKE, n_max + 1) == -2
    assert "SSU_MAX_PAIRS" in ssu.ssu_last_error()


def test_empty_calls_are_noops(ssu):
    c = _cache(ssu)
    assert ssu.ssu_replay_step(c, _step(ssu, batch=0)) == 0
    assert ssu.ssu_flush(c, FAKE, FAKE, FAKE, 0) == 0
    assert ssu.ssu_init_state(c, FAKE, 0, FAKE, 0) == 0
    assert ssu.ssu_flush(c, FAKE, FAKE, FAKE, -1) == -1
    assert ssu.ssu_flush(c, None, FAKE, FAKE, 2) == -1


def test_product_does_not_import_the_oracle():
    """The library package never reaches the CPU oracle."""
    pkg = os.path.join(ROOT, "speculative_replay_state_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h", ".cuh")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.lower(), f


def test_step_desc_keeps_its_tensors_alive(ssu):
    """The step descriptor holds raw pointers; it must keep the tensors behind
    them (the split workspace among them) alive until it is dropped."""
    import gc
    import weakref
    import torch
    ws = torch.empty(16)
    t = torch.zeros(4, dtype=torch.int32)
    ref = weakref.ref(ws)
    d = ssu.make_step_desc(1, 1, t, t, None, t, t, t, t, t, t, t, t, workspace=ws)
    del ws
    gc.collect()
    assert ref() is not None and d.workspace_bytes == 64
    del d
    gc.collect()
    assert ref() is None


def test_binding_refuses_host_tensors(ssu):
    """The torch front end never hands a host pointer to the library: a cache
    or step tensor that is not on the GPU is a ValueError before any call."""
    import torch
    u8 = lambda n: torch.zeros(4, n, dtype=torch.uint8)
    dc = ssu.DeviceCache(4, 16, 2, 16, "bf16", u8(16 * 64 * 128 * 2), None, u8(16 * 16 * 64 * 2),
                         u8(2 * 16 * 128 * 2), u8(16 * 16 * 4), torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="device tensor"):
        dc.desc()
    t = torch.zeros(64, dtype=torch.int32)
    d = ssu.make_step_desc(1, 1, t, t, None, t, t, t, t, t, t, t, t)
    with pytest.raises(ValueError, match="device tensor"):
        ssu.check_step_tensors(dc, d)
    with pytest.raises(ValueError, match="device tensor"):
        ssu.replay_step(dc, d)
    with pytest.raises(ValueError, match="device tensor"):
        ssu.flush(dc, t, t, t)
