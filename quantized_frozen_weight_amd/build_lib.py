"""Build libqlora.so (all HIP sources under csrc/) for gfx950 with hipcc.

    python -m quantized_frozen_weight_amd.build_lib

The library is written next to this file so that it travels with the source
tree; it is rebuilt every time this runs.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libqlora.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no hand-written or compiler-formed packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE float32 on the device: keep denormals, correctly rounded divide
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # MFMA accumulators in ordinary VGPRs: no copies between the
    # accumulation registers and VGPRs inside the main loops
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, out: str = LIB_PATH, defines=()) -> str:
    """Compile every csrc/*.hip (one hipcc per source, in parallel) and link
    them into one shared library at ``out``.

    ``defines`` are extra -D flags (tuning knobs)."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    flags = [*HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC]

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            sys.stderr.write(proc.stdout + proc.stderr)
            raise RuntimeError(f"hipcc failed ({proc.returncode}): {cmd[-1]}")

    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *flags, "-c", src, "-o", obj])
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(run, cmds))
    tmp = out + ".tmp"
    run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    shutil.rmtree(objdir, ignore_errors=True)
    return out


# Host code of the library under AddressSanitizer and
# UndefinedBehaviorSanitizer (the device code is built as usual, without
# them).
SANITIZE_HOST = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
]


def llvm_bin(tool: str) -> str:
    path = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", tool)
    if not os.path.exists(path):
        path = os.path.join("/opt/rocm/lib/llvm/bin", tool)
    return path


def build_host_sanitized(driver: str, out: str, verbose: bool = False) -> str:
    """Build the executable ``out`` from the C program ``driver`` and the
    library's sources compiled for the host only, with the sanitizers above
    on every host object (the driver included)."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = out + ".objs"
    os.makedirs(objdir, exist_ok=True)
    flags = [*HIPCC_FLAGS, "-g", "-Xarch_host", "-fno-omit-frame-pointer", *SANITIZE_HOST,
             "-I", INCLUDE, "-I", CSRC]

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            sys.stderr.write(proc.stdout + proc.stderr)
            raise RuntimeError(f"build failed ({proc.returncode}): {cmd[-1]}")

    cmds, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *flags, "-c", src, "-o", obj])
    dobj = os.path.join(objdir, "driver.o")
    cmds.append([llvm_bin("clang"), "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                 "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                 "-Wall", "-Werror", "-I", INCLUDE, "-c", driver, "-o", dobj])
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(run, cmds))
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "lib")
    run([llvm_bin("clang++"), "-fsanitize=address,undefined", dobj, *objs, "-o", out,
         f"-L{rocm_lib}", f"-Wl,-rpath,{rocm_lib}", "-lamdhip64"])
    shutil.rmtree(objdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB_PATH)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    a = ap.parse_args()
    print(build(verbose=True, out=a.out, defines=a.defines))
