"""Build libmoe_ep.so (the gfx950 dispatch/combine library) in-tree with hipcc.

    python -m combine_token_dest_amd.build

Every call compiles from source; the library lands next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_ep.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep hipcc from fusing float adds into v_pk_add_f32.
# kernarg preload: the leading scalar kernel arguments arrive in scalar
# registers at wave launch instead of through a load from the argument block.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-kernarg-preload-count=16"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
          f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build step failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile the kernels for gfx950 and the host API, link LIB_PATH."""
    with tempfile.TemporaryDirectory(prefix="moe_ep_build_") as tmp:
        k_obj = os.path.join(tmp, "moe_ep_kernels.o")
        a_obj = os.path.join(tmp, "moe_ep_api.o")
        p_obj = os.path.join(tmp, "moe_ep_plan.o")
        lib_tmp = os.path.join(tmp, LIB_NAME)
        steps = [
            [HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c",
             os.path.join(CSRC, "moe_ep_kernels.hip"), "-o", k_obj],
            [HIPCC, *COMMON, "-c", os.path.join(CSRC, "moe_ep_api.cpp"), "-o", a_obj],
            [HIPCC, *COMMON, "-c", os.path.join(CSRC, "moe_ep_plan.cpp"), "-o", p_obj],
            [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", k_obj, a_obj, p_obj, "-o", lib_tmp],
        ]
        for cmd in steps:
            out = _run(cmd)
            if verbose and out.strip():
                print(out)
        shutil.move(lib_tmp, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


C_ROUND_SRC = os.path.join(ROOT, "tests", "host", "c_round.c")
C_ROUND_BIN = os.path.join(ROOT, "tests", "host", "c_round")


def build_c_round() -> str:
    """Compile tests/host/c_round.c, a round through the C ABI alone (plain
    C99 with the HIP runtime's C API), linked against LIB_PATH."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    tmp = C_ROUND_BIN + ".tmp"
    _run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          f"-I{rocm}/include", f"-I{INCLUDE}", C_ROUND_SRC, f"-L{PKG_DIR}", "-lmoe_ep",
          f"-L{rocm}/lib", "-lamdhip64", "-lm",
          "-Wl,-rpath,$ORIGIN/../../combine_token_dest_amd", f"-Wl,-rpath,{rocm}/lib", "-o", tmp])
    os.replace(tmp, C_ROUND_BIN)
    return C_ROUND_BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_c_round())
