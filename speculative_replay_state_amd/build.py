"""Build libssu.so (gfx950) in-tree with hipcc.

    python speculative_replay_state_amd/build.py

(run as a script: importing the package fails until the library exists)

Compiles the device code (csrc/ssu_kernels.cuh through ssu_kernels_inst.hip,
once per state type, in parallel), the dispatch (csrc/ssu_launch.cpp) and the
host entry points (csrc/ssu_api.cpp), and links them into
speculative_replay_state_amd/libssu.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssu.so")
ARCH = os.environ.get("SSU_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libssu needs ROCm's hipcc to build")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n  %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="ssu_build_") as tmp:
        objs, jobs = [], []
        # the kernels once per state type (fp32, bf16, fp16, fp8, nvfp4), compiled in parallel
        for st in range(5):
            o = os.path.join(tmp, "ssu_kernels_%d.o" % st)
            objs.append(o)
            jobs.append([hipcc, "--offload-arch=" + ARCH, *COMMON, "-DSSU_INST_ST=%d" % st, "-c",
                         os.path.join(CSRC, "ssu_kernels_inst.hip"), "-o", o])
        for src in ("ssu_launch.cpp", "ssu_api.cpp"):
            o = os.path.join(tmp, src.replace(".cpp", ".o"))
            objs.append(o)
            jobs.append([hipcc, "--offload-arch=" + ARCH, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src),
                         "-o", o])
        with concurrent.futures.ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 1)) as ex:
            outs = list(ex.map(_run, jobs))
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        outs.append(_run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib, *objs]))
        os.replace(tmp_lib, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
