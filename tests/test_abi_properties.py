"""Host validation as a property: random cache and step descriptors, and the
library's answer checked against the requirements include/ssu.h states.

The descriptors are drawn near the edges of every documented requirement
(alignment, NULL pointers, slot strides, dtypes, ring_len, max_seqlen, the
fused flush with SPLIT).  For each one the test lists, from its own reading
of the header, which requirements are broken and which error codes the
header allows for each.  Then:
  - no broken requirement: ssu_resolve_algo returns the algorithm the step
    runs (an explicit MONOLITH or SPLIT, a fused step MONOLITH, else AUTO's
    work-unit threshold), and ssu_workspace_size is positive;
  - broken requirements: the return is the code of one of them and a message
    is set, ssu_replay_step and ssu_replay_step_noalloc return the same code,
    and, where the cache itself is broken, so do ssu_flush and ssu_init_state
    while ssu_workspace_size is 0.
No call here launches a kernel: every entry point that could launch is only
called once ssu_resolve_algo has rejected the same descriptors (the checks are
pure functions of them), or with batch 0 (a no-op).  The pointers are never
dereferenced.
"""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

OK, INVALID, UNSUPPORTED = 0, -1, -2
F32, BF16, F16, FP8, NVFP4 = 0, 1, 2, 3, 4
AUTO, MONOLITH, SPLIT = 0, 1, 2
BASE = 0x100000  # 256-byte aligned, never dereferenced

# bytes of one head's checkpoint (64 x 128 values) by state dtype
HEAD_BYTES = {F32: 64 * 128 * 4, BF16: 64 * 128 * 2, F16: 64 * 128 * 2, FP8: 64 * 128, NVFP4: 64 * 128 // 2}


@pytest.fixture(scope="module")
def ssu():
    import speculative_replay_state_amd as m
    return m


def mostly(good, bad):
    """`good` in 49 draws of 50, else `bad`: most descriptors then break
    one requirement or none, and every requirement is broken on its own."""
    return st.integers(0, 49).flatmap(lambda n: bad if n == 25 else good)


def ptr(align, optional=False):
    """A pointer aligned to `align` (or NULL when `optional`), else NULL or
    misaligned."""
    good = st.integers(0, 64).map(lambda i: BASE + i * 256 + (0 if align == 16 else 4 * (i % 4)))
    if optional:
        good = st.one_of(st.none(), good)
    return mostly(good, st.sampled_from([None, BASE + 1, BASE + 2, BASE + 8]))


def stride(need):
    """A slot stride: the packed size `need` rounded up to 16 bytes, plus
    padding; else too small or not a multiple of 16."""
    up = (need + 15) // 16 * 16
    return mostly(st.sampled_from([0, 16, 64, 1024]), st.sampled_from([-16, -8, 8, -up])).map(
        lambda pad: up + pad)


@st.composite
def cache_fields(draw):
    c = {}
    c["num_slots"] = draw(mostly(st.sampled_from([1, 2, 9, 1000]), st.sampled_from([0, -1])))
    c["ngroups"] = draw(mostly(st.sampled_from([1, 2, 4, 8]), st.sampled_from([0, 3, 16])))
    c["nheads"] = draw(mostly(st.sampled_from([1, 2, 3, 4, 6, 12, 32, 96]).map(lambda m: m * c["ngroups"]),
                              st.sampled_from([0, -4, 1, 2, 5, 7, 9])))
    c["headdim"] = draw(mostly(st.just(64), st.sampled_from([32, 128, 0])))
    c["dstate"] = draw(mostly(st.just(128), st.sampled_from([64, 256])))
    c["ring_len"] = draw(mostly(st.integers(1, 32), st.sampled_from([-1, 0, 33, 40])))
    sd = c["state_dtype"] = draw(mostly(st.sampled_from([F32, BF16, F16, FP8, NVFP4]), st.sampled_from([7, -1])))
    c["io_dtype"] = draw(mostly(st.just(BF16), st.sampled_from([F32, F16, FP8])))
    for k in ("state", "x_cache", "B_cache", "dt_cache"):
        c[k] = draw(ptr(16))
    c["ring_start"] = draw(ptr(4))
    c["status"] = draw(ptr(4, optional=True))
    c["state_scale"] = draw(ptr(16, optional=sd not in (FP8, NVFP4)))
    c["state_gscale"] = draw(ptr(16, optional=sd != NVFP4))
    # recur_state: required with nvfp4, optional with fp8, else absent
    if sd == NVFP4:
        c["recur_state"] = draw(ptr(16))
    elif sd == FP8:
        c["recur_state"] = draw(ptr(16, optional=True))
    else:
        c["recur_state"] = draw(mostly(st.none(), st.just(BASE)))
    # strides drawn around what a well-formed cache of these sizes needs
    H, G = max(c["nheads"], 1), max(c["ngroups"], 1)
    L = max(c["ring_len"], 1)
    eb = HEAD_BYTES.get(sd, 64 * 128 * 2)
    c["state_slot_stride"] = draw(stride(H * eb))
    c["scale_slot_stride"] = draw(stride(H * (512 if sd == NVFP4 else 64 * 4)))
    c["gscale_slot_stride"] = draw(stride((1 + H) * 4))
    c["x_slot_stride"] = draw(stride(H * L * 64 * 2))
    c["B_slot_stride"] = draw(stride(G * L * 128 * 2))
    c["dt_slot_stride"] = draw(stride(H * L * 4))
    c["recur_slot_stride"] = draw(stride(H * 64 * 128 * 2))
    return c


@st.composite
def step_fields(draw, ring_len):
    s = {}
    s["batch"] = draw(mostly(st.sampled_from([0, 1, 3, 64, 2049, 1 << 20]), st.just(-1)))
    s["max_seqlen"] = draw(mostly(st.integers(1, max(1, min(16, ring_len))), st.integers(-1, 34)))
    for k in ("x", "B", "C", "out"):
        s[k] = draw(ptr(16))
    for k in ("dt", "A", "D", "dt_bias", "slot_idx", "prev_num_accepted"):
        s[k] = draw(ptr(4))
    s["cu_seqlens"] = draw(ptr(4, optional=True))
    s["num_fold"] = draw(ptr(4, optional=True))
    s["z"] = draw(ptr(16, optional=True))
    s["out_dtype"] = draw(mostly(st.sampled_from([BF16, F32]), st.sampled_from([F16, FP8, 9])))
    s["algo"] = draw(mostly(st.sampled_from([AUTO, MONOLITH, SPLIT]), st.sampled_from([9, -1])))
    return s


def aligned(p, a):
    return p % a == 0


def cache_violations(c):
    """(requirement, allowed codes) for every requirement of the cache
    description that `c` breaks, as the header states them."""
    v = []
    either = {INVALID, UNSUPPORTED}
    if c["num_slots"] < 1 or c["nheads"] < 1 or c["ngroups"] < 1:
        v.append(("positive sizes", {INVALID}))
    elif c["nheads"] % c["ngroups"]:
        v.append(("nheads % ngroups", {INVALID}))
    if c["headdim"] != 64 or c["dstate"] != 128:
        v.append(("headdim 64, dstate 128", {UNSUPPORTED}))
    if not 1 <= c["ring_len"] <= 32:
        v.append(("1 <= ring_len <= 32", either))
    sd = c["state_dtype"]
    if sd not in HEAD_BYTES:
        v.append(("state_dtype", {INVALID}))
    if c["io_dtype"] != BF16:
        v.append(("io_dtype bf16", either))
    for k in ("state", "x_cache", "B_cache", "dt_cache", "ring_start"):
        if c[k] is None:
            v.append((k + " not NULL", {INVALID}))
    if sd in (FP8, NVFP4) and c["state_scale"] is None:
        v.append(("state_scale", {INVALID}))
    if sd == NVFP4 and c["state_gscale"] is None:
        v.append(("state_gscale", {INVALID}))
    if sd == NVFP4 and c["recur_state"] is None:
        v.append(("nvfp4 requires recur_state", {UNSUPPORTED}))
    if c["recur_state"] is not None and sd not in (FP8, NVFP4):
        v.append(("recur_state requires fp8 or nvfp4", {UNSUPPORTED}))
    for k in ("state", "x_cache", "B_cache", "dt_cache", "state_scale", "state_gscale", "recur_state"):
        if c[k] is not None and not aligned(c[k], 16):
            v.append((k + " 16-byte aligned", {INVALID}))
    for k in ("ring_start", "status"):  # i32 arrays
        if c[k] is not None and not aligned(c[k], 4):
            v.append((k + " 4-byte aligned", {INVALID}))
    # slot strides of the tensors in use: at least one packed slot page, and
    # a multiple of 16 (the page layouts at ssu_cache)
    if c["nheads"] >= 1 and c["ngroups"] >= 1 and c["ring_len"] >= 1 and sd in HEAD_BYTES:
        H, G, L = c["nheads"], c["ngroups"], c["ring_len"]
        used = [("state", c["state_slot_stride"], H * HEAD_BYTES[sd]),
                ("x_cache", c["x_slot_stride"], H * L * 64 * 2),
                ("B_cache", c["B_slot_stride"], G * L * 128 * 2),
                ("dt_cache", c["dt_slot_stride"], H * L * 4)]
        if sd == FP8:
            used.append(("state_scale", c["scale_slot_stride"], H * 64 * 4))
        if sd == NVFP4:
            used.append(("state_scale", c["scale_slot_stride"], H * 512))
            used.append(("state_gscale", c["gscale_slot_stride"], (1 + H) * 4))
        if c["recur_state"] is not None:
            used.append(("recur_state", c["recur_slot_stride"], H * 64 * 128 * 2))
        for name, s, need in used:
            if s < need or s % 16:
                v.append((name + " slot stride", {INVALID}))
    return v


def step_violations(c, s):
    v = []
    either = {INVALID, UNSUPPORTED}
    if s["batch"] < 0:
        v.append(("batch >= 0", {INVALID}))
    if s["max_seqlen"] < 1:
        v.append(("max_seqlen >= 1", {INVALID}))
    elif s["max_seqlen"] > c["ring_len"]:
        v.append(("max_seqlen <= ring_len", {INVALID}))
    elif s["max_seqlen"] > 16:
        v.append(("max_seqlen <= 16", either))
    if s["batch"] <= 0:
        return v  # batch 0 is a no-op: the step's tensors are not looked at
    if s["batch"] * c["nheads"] > (1 << 24) - 1:
        v.append(("batch * nheads <= SSU_MAX_PAIRS", {UNSUPPORTED}))
    for k in ("slot_idx", "prev_num_accepted", "x", "B", "C", "dt", "A", "D", "dt_bias", "out"):
        if s[k] is None:
            v.append((k + " not NULL", {INVALID}))
    if s["out_dtype"] not in (BF16, F32):
        v.append(("out_dtype", either))
    for k in ("x", "B", "C", "out", "z"):
        if s[k] is not None and not aligned(s[k], 16):
            v.append((k + " 16-byte aligned", {INVALID}))
    for k in ("dt", "A", "D", "dt_bias", "slot_idx", "prev_num_accepted", "cu_seqlens", "num_fold"):
        if s[k] is not None and not aligned(s[k], 4):
            v.append((k + " 4-byte aligned", {INVALID}))
    if s["algo"] not in (AUTO, MONOLITH, SPLIT):
        v.append(("algo", {INVALID}))
    elif s["algo"] == SPLIT and s["num_fold"] is not None:
        v.append(("num_fold runs in the monolith", {UNSUPPORTED}))
    return v


def build(ssu, cache, step):
    c = ssu.SsuCache()
    for k, val in cache.items():
        setattr(c, k, val)
    s = ssu.SsuStep()
    for k, val in step.items():
        setattr(s, k, val)
    return c, s


@settings(max_examples=3000, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])
@given(cache_step=cache_fields().flatmap(lambda c: st.tuples(st.just(c), step_fields(c["ring_len"]))),
       threshold=st.sampled_from([1, 64, 4096, 2 ** 63 - 1]))
def test_validation_matches_the_header(ssu, cache_step, threshold):
    cache, step = cache_step
    c, s = build(ssu, cache, step)
    cv = cache_violations(cache)
    sv = step_violations(cache, step) if not cv else []
    old = ssu.ssu_set_split_threshold(threshold)
    try:
        rc = ssu.ssu_resolve_algo(c, s)
        msg = ssu.ssu_last_error()
    finally:
        ssu.ssu_set_split_threshold(old)
    ws = ssu.ssu_workspace_size(c, 1, 1)
    if cv:
        assert rc in set().union(*(codes for _, codes in cv)), (rc, msg, cv)
        assert msg and ssu.ssu_last_error() == msg  # the cache check again
        assert ws == 0
        # every entry point checks the cache first, the same way
        assert ssu.ssu_flush(c, BASE, BASE, BASE, 1) == rc
        assert ssu.ssu_init_state(c, BASE, 0, BASE, 1) == rc
        assert ssu.ssu_replay_step(c, s) == rc
        assert ssu.ssu_replay_step_noalloc(c, s) == rc
        return
    assert ws > 0 and ssu.ssu_last_error() == "", ssu.ssu_last_error()
    if sv:
        assert rc in set().union(*(codes for _, codes in sv)), (rc, msg, sv)
        assert msg
        assert ssu.ssu_replay_step(c, s) == rc
        assert ssu.ssu_replay_step_noalloc(c, s) == rc
        return
    assert rc >= 0, (rc, msg)
    assert msg == ""
    if step["algo"] in (MONOLITH, SPLIT):
        want = step["algo"]
    elif step["num_fold"] is not None:
        want = MONOLITH  # a fused step runs in the monolith
    else:
        want = SPLIT if step["batch"] * cache["nheads"] >= threshold else MONOLITH
    assert rc == want
    if step["batch"] == 0:
        assert ssu.ssu_replay_step(c, s) == OK  # a no-op: no launch


@settings(max_examples=400, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(cache=cache_fields(), b1=st.integers(0, 4096), b2=st.integers(0, 4096), t=st.integers(0, 16))
def test_workspace_size_properties(ssu, cache, b1, b2, t):
    """SPLIT's scratch holds one fp32 C.B product per (entry, group, new
    token, ring position): at least batch * ngroups * T * ring_len * 4 bytes,
    additive over entries, 0 for an empty step, an invalid cache or a step
    past the header's limits (T > min(16, ring_len), batch * nheads >
    SSU_MAX_PAIRS)."""
    c, _ = build(ssu, cache, {})
    w = lambda b, tt: ssu.ssu_workspace_size(c, b, tt)
    if cache_violations(cache):
        assert w(b1, t) == 0
        return
    G, L = cache["ngroups"], cache["ring_len"]
    if t > min(16, L):
        assert w(b1, t) == 0 and ssu.ssu_last_error()
        return
    assert w(ssu.SSU_MAX_PAIRS // cache["nheads"] + 1, t) == 0 and "SSU_MAX_PAIRS" in ssu.ssu_last_error()
    assert w(b1, t) >= b1 * G * t * L * 4
    assert w(b1 + b2, t) == w(b1, t) + w(b2, t)
    assert w(0, t) == 0 and w(b1, 0) == 0
    assert w(b1, t) % 16 == 0  # a workspace slice per entry stays 16-byte aligned
    assert w(-1, t) == 0 and w(b1, -1) == 0
