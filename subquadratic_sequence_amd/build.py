"""Builds libhyena.so (the C-ABI library of the HIP kernels) for gfx950 in-tree.

    python -m subquadratic_sequence_amd.build

Every source under csrc/ is compiled with hipcc, then linked into
subquadratic_sequence_amd/libhyena.so. The packed-fp32 target feature is
switched off for all device code.

    python -m subquadratic_sequence_amd.build --abi-check

also links tests/abi_check.c into _build/abi_check: the host-side entry points
(csrc/api.cpp, csrc/nd_api.cpp, csrc/noalloc.hip) rebuilt with AddressSanitizer
and UndefinedBehaviorSanitizer on their host code only (every finding aborts),
with the kernels' objects of the plain build. It runs on the CPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libhyena.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_INC = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "include")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-signed-zeros",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# Host-side entry points: argument validation and size arithmetic live here.
SANITIZED = ["api.cpp", "nd_api.cpp", "noalloc.hip"]
# Sanitizers act on the host pass only (device code is built as usual).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
CHECK_SRC = os.path.join(os.path.dirname(HERE), "tests", "abi_check.c")
CHECK_OUT = os.path.join(OBJ_DIR, "abi_check")


def build_abi_check(verbose: bool = False) -> str:
    """Links the sanitized ABI check; the kernels' objects come from build()."""
    plain = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    kernels = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in plain
               if os.path.basename(s) not in SANITIZED]
    if not all(os.path.exists(o) for o in kernels):
        build()
    objs = []
    for name in SANITIZED:
        obj = os.path.join(OBJ_DIR, name + ".san.o")
        cmd = [HIPCC, *FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, name), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized build failed for {name}:\n{r.stderr}")
        objs.append(obj)
    inc = os.path.join(os.path.dirname(HERE), "include")
    main_obj = os.path.join(OBJ_DIR, "abi_check.o")
    cmd = [HIPCC, "-x", "c", "-std=c11", "-Wall", "-Werror", *SAN_FLAGS, "-I", inc, "-I", ROCM_INC,
           "-D__HIP_PLATFORM_AMD__", "-c", CHECK_SRC, "-o", main_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"abi_check.c failed to compile:\n{r.stderr}")
    cmd = [HIPCC, f"--offload-arch={ARCH}", *SAN_FLAGS, "-o", CHECK_OUT, main_obj, *objs, *kernels]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"abi_check link failed:\n{r.stderr}")
    if verbose:
        print(f"built {CHECK_OUT}")
    return CHECK_OUT


if __name__ == "__main__":
    build(verbose=True)
    if "--abi-check" in sys.argv[1:]:
        build_abi_check(verbose=True)
    sys.exit(0)
