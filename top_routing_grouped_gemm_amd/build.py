"""Build ``libmoe.so`` (the HIP kernels + C ABI of include/moe.h) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature flag and says so; that is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


C_EXAMPLE = os.path.join(ROOT, "tests", "c_abi", "forward.c")
C_EXAMPLE_BIN = os.path.join(ROOT, "tests", "c_abi", "forward")


def c_example_cmd(src: str, out: str) -> list:
    """gcc line of the plain-C caller of the ABI (tests/c_abi/forward.c), linked to libmoe.so by a relative rpath."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rel = os.path.relpath(HERE, os.path.dirname(out))
    return ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
            f"-I{rocm}/include", src, f"-L{HERE}", "-lmoe", f"-L{rocm}/lib", "-lamdhip64",
            f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{rocm}/lib", "-o", out]


def build_c_example(out: str = C_EXAMPLE_BIN) -> str:
    res = subprocess.run(c_example_cmd(C_EXAMPLE, out), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_example())
