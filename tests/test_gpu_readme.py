"""The usage examples in README.md run as written on the GPU: the Python one
through the binding, the C one compiled by gcc against include/ssu.h and
linked to libssu.so and the HIP runtime."""
import os
import re
import shutil
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_readme_example_runs():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    print("README example", flush=True)
    exec(compile(blocks[0], "README.md", "exec"), {})


def test_readme_c_example_runs(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```c\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    src = tmp_path / "example.c"
    src.write_text(blocks[0])
    lib = os.path.join(ROOT, "speculative_replay_state_amd")
    exe = tmp_path / "example"
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src), "-o", str(exe),
                    "-L", lib, "-lssu", "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath," + lib + ":/opt/rocm/lib"],
                   check=True, capture_output=True, text=True)
    print("README C example", flush=True)
    p = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.startswith("status 0") and "nan" not in p.stdout.lower(), p.stdout
