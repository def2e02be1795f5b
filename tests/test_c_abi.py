"""The C ABI from a plain C99 program (tests/c_abi_smoke.c): the header
compiles as C, the program links against the library and the HIP runtime
(CPU), and on the GPU it reproduces the value rows bit for bit through exact
pixel-centre gathers and gets MSDA_ERR_UNSUPPORTED for a 12-byte head row."""
import os
import shutil
import subprocess

import pytest

from scale_deformable_attention_02_amd import _build, binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_smoke.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(out_dir):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("gcc or the HIP runtime headers are not installed")
    if not os.path.exists(binding.library_path()):
        _build.build()
    lib_dir = os.path.dirname(binding.library_path())
    exe = os.path.join(str(out_dir), "c_abi_smoke")
    cmd = [gcc, "-std=c99", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", lib_dir, "-lmsda", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_compiles_and_links(tmp_path):
    assert os.access(_compile(tmp_path), os.X_OK)


@pytest.mark.gpu
def test_c_program_runs_on_the_gpu(tmp_path):
    exe = _compile(tmp_path)
    print("[c-abi] running the C caller", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
