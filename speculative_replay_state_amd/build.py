"""Build libssu.so (gfx950) in-tree with hipcc.

    python -m speculative_replay_state_amd.build

Compiles csrc/ssu_kernels.hip (device code) and csrc/ssu_api.cpp (host entry
points) and links them into speculative_replay_state_amd/libssu.so.
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
        k_obj = os.path.join(tmp, "ssu_kernels.o")
        a_obj = os.path.join(tmp, "ssu_api.o")
        jobs = [
            [hipcc, "--offload-arch=" + ARCH, *COMMON, "-c", os.path.join(CSRC, "ssu_kernels.hip"),
             "-o", k_obj],
            [hipcc, "--offload-arch=" + ARCH, *COMMON, "-x", "hip", "-c",
             os.path.join(CSRC, "ssu_api.cpp"), "-o", a_obj],
        ]
        with concurrent.futures.ThreadPoolExecutor(2) as ex:
            outs = list(ex.map(_run, jobs))
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        outs.append(_run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib, k_obj, a_obj]))
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
