"""The C ABI as a C compiler sees it.

include/ssu.h is compiled as C11 by gcc (no HIP compiler) into a small
program linked against libssu.so.  The program prints the size and every
field offset of ssu_cache and ssu_step, the enum values and the macros, and
the answers of two host-only calls on a descriptor it builds itself.  The
Python binding's ctypes structures and constants must agree with all of it,
or the binding would hand the library misplaced fields.  No kernel runs.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CONSTANTS = ["SSU_F32", "SSU_BF16", "SSU_F16", "SSU_FP8_E4M3", "SSU_NVFP4", "SSU_ALGO_AUTO", "SSU_ALGO_MONOLITH",
             "SSU_ALGO_SPLIT", "SSU_OK", "SSU_ERR_INVALID", "SSU_ERR_UNSUPPORTED", "SSU_ERR_HIP", "SSU_ERR_WORKSPACE",
             "SSU_STATUS_BAD_PNAT", "SSU_STATUS_BAD_FOLD", "SSU_STATUS_BAD_SEQLEN", "SSU_STATUS_BAD_RING",
             "SSU_MAX_PAIRS", "SSU_NOALLOC_SCRATCH_BYTES"]


@pytest.fixture(scope="module")
def ssu():
    import speculative_replay_state_amd as m
    return m


@pytest.fixture(scope="module")
def c_report(ssu, tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    d = tmp_path_factory.mktemp("abi_c")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ssu.h"', 'int main(void) {']
    for cname, ctype in (("ssu_cache", ssu.SsuCache), ("ssu_step", ssu.SsuStep)):
        lines.append('  printf("size %s %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in ctype._fields_:
            lines.append('  printf("off %s.%s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    for k in CONSTANTS:
        lines.append('  printf("const %s %%lld\\n", (long long)(%s));' % (k, k))
    # the defaults of tests/test_abi.py's valid descriptors, built in C
    lines += [
        '  char *fake = (char *)0x10000;',
        '  ssu_cache c = {0};',
        '  c.num_slots = 8; c.nheads = 16; c.ngroups = 2; c.headdim = 64; c.dstate = 128; c.ring_len = 16;',
        '  c.state_dtype = SSU_BF16; c.io_dtype = SSU_BF16;',
        '  c.state = fake; c.state_slot_stride = 16 * 64 * 128 * 2;',
        '  c.x_cache = fake; c.x_slot_stride = 16 * 16 * 64 * 2;',
        '  c.B_cache = fake; c.B_slot_stride = 2 * 16 * 128 * 2;',
        '  c.dt_cache = (float *)fake; c.dt_slot_stride = 16 * 16 * 4;',
        '  c.ring_start = (int32_t *)fake;',
        '  ssu_step s = {0};',
        '  s.batch = 4; s.max_seqlen = 4; s.slot_idx = (const int32_t *)fake; s.prev_num_accepted = s.slot_idx;',
        '  s.x = fake; s.B = fake; s.C = fake; s.dt = (const float *)fake; s.A = s.dt; s.D = s.dt;',
        '  s.dt_bias = s.dt; s.out = fake; s.out_dtype = SSU_BF16; s.algo = SSU_ALGO_SPLIT;',
        '  printf("call workspace %zu\\n", ssu_workspace_size(&c, 4, 4));',
        '  printf("call resolve %d\\n", ssu_resolve_algo(&c, &s));',
        '  s.max_seqlen = 17;',
        '  printf("call resolve_bad %d\\n", ssu_resolve_algo(&c, &s));',
        '  return 0;', '}']
    src = d / "abi.c"
    src.write_text("\n".join(lines) + "\n")
    exe = d / "abi"
    libdir = os.path.dirname(ssu.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src), "-o", str(exe),
                    "-L", libdir, "-lssu", "-Wl,-rpath," + libdir], check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    rep = {}
    for line in out.splitlines():
        kind, key, val = line.split()
        rep[(kind, key)] = int(val)
    return rep


def test_struct_layout_matches_ctypes(ssu, c_report):
    for cname, ctype in (("ssu_cache", ssu.SsuCache), ("ssu_step", ssu.SsuStep)):
        assert c_report[("size", cname)] == ctypes.sizeof(ctype), cname
        for f, _ in ctype._fields_:
            assert c_report[("off", "%s.%s" % (cname, f))] == getattr(ctype, f).offset, (cname, f)


def test_constants_match_the_binding(ssu, c_report):
    for k in CONSTANTS:
        assert c_report[("const", k)] == getattr(ssu, k), k


def test_c_caller_gets_the_binding_answers(ssu, c_report):
    from tests.test_abi import _cache, _step
    c = _cache(ssu)
    assert c_report[("call", "workspace")] == ssu.ssu_workspace_size(c, 4, 4) > 0
    assert c_report[("call", "resolve")] == ssu.ssu_resolve_algo(c, _step(ssu)) == ssu.SSU_ALGO_SPLIT
    assert c_report[("call", "resolve_bad")] == ssu.SSU_ERR_INVALID
