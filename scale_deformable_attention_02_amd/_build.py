"""Build the HIP library ``libmsda.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmsda.so")
SOURCES = [os.path.join(CSRC, "msda_api.hip"), os.path.join(CSRC, "msda_api_fused.hip"),
           os.path.join(CSRC, "msda_api_pruned.hip"), os.path.join(CSRC, "msda_backward_api.hip"),
           os.path.join(CSRC, "msda_linear.hip"), os.path.join(CSRC, "msda_order.hip"),
           os.path.join(CSRC, "msda_calib.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "msda_device.hpp"), os.path.join(CSRC, "msda_backward.hpp"),
                     os.path.join(CSRC, "msda_forward_impl.hpp"),
                     os.path.join(CSRC, "msda_host.hpp"),
                     os.path.join(INCLUDE, "msda.h"), os.path.join(INCLUDE, "msda_calib.h")]

ARCH = "gfx950"


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def compile_flags(extra=()):
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        # packed fp32 arithmetic stays off (v_pk_{add,mul,fma}_f32 are not used)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        *extra,
    ]


def build(verbose: bool = False, extra=()) -> str:
    """Compile ``libmsda.so`` (always rebuilds); returns its path.

    Each translation unit is compiled by its own hipcc process (in parallel),
    then the objects are linked."""
    import concurrent.futures
    import tempfile

    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="msda_build_") as work:
        objs = [os.path.join(work, os.path.splitext(os.path.basename(src))[0] + ".o")
                for src in SOURCES]
        cmds = [[hipcc(), *compile_flags(extra), "-c", "-o", obj, src]
                for src, obj in zip(SOURCES, objs)]
        cmds.append([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])

        def run(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            proc = subprocess.run(cmd, capture_output=True, text=True)
            if proc.returncode != 0:
                raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr}")

        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
            list(pool.map(run, cmds[:-1]))
        run(cmds[-1])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
