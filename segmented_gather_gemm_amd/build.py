"""Compile libsgg_lora.so (host planner + gfx950 HIP kernels) and the CPython
call module over it, in the package directory."""

import os
import subprocess
import sys
import sysconfig

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsgg_lora.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
CALLMOD = os.path.join(PKG, "_sggcall" + sysconfig.get_config_var("EXT_SUFFIX"))
SOURCES = ["plan.cpp", "tiling.cpp", "plan_device.hip", "shrink.hip", "shrink_gemm.hip",
           "expand.hip", "fused.hip", "moe.hip", "lora_api.hip"]
ARCH = os.environ.get("SGG_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose, what):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"{what} failed with status {res.returncode}")


def build(verbose=False):
    """Build the shared library and the CPython call module; always
    recompiles (one hipcc per source, in parallel, then one link).  Returns
    the library's path."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]

    def compile_one(i):
        _run([hipcc()] + HIPCC_FLAGS + ["-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]],
             verbose, f"hipcc {SOURCES[i]}")

    workers = max(1, min(len(SOURCES), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(workers) as pool:
        list(pool.map(compile_one, range(len(SOURCES))))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose,
         "hipcc link")
    os.replace(tmp, LIB)
    # integer-argument entry points for the hot calls, linked to the library
    tmp = CALLMOD + ".tmp"
    _run([os.environ.get("CC", "gcc"), "-O2", "-shared", "-fPIC", "-Wall",
          "-I", sysconfig.get_paths()["include"], "-I", INCLUDE,
          os.path.join(CSRC, "pycall.c"), "-L", PKG, "-lsgg_lora",
          "-Wl,-rpath,$ORIGIN", "-o", tmp], verbose, "cc")
    os.replace(tmp, CALLMOD)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
