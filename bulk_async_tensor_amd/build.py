"""Build libep.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m bulk_async_tensor_amd.build`` or ``build()`` from Python.
Objects go to ``bulk_async_tensor_amd/_build/``; the library is written to
``bulk_async_tensor_amd/libep.so``.  Every call recompiles.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libep.so")
SOURCES = ["ep_api.hip", "layout.hip", "dispatch.hip", "dispatch_rows.hip", "combine.hip", "combine_reduce.hip",
           "layout_dispatch.hip", "probe.hip"]
ARCH = "gfx950"


# The sources each measured kernel and its launch geometry are compiled from
# (the C ABI in ep_api.hip only validates arguments and forwards them).
KERNEL_SOURCES = {
    "layout": ["layout.hip", "ep_device.hpp", "ep_internal.hpp"],
    "dispatch": ["dispatch.hip", "dispatch_rows.hip", "row_io.hpp", "ep_device.hpp", "ep_internal.hpp"],
    "combine": ["combine.hip", "row_io.hpp", "ep_device.hpp", "ep_internal.hpp"],
    "combine_reduce": ["combine_reduce.hip", "row_io.hpp", "ep_device.hpp", "ep_internal.hpp"],
    "layout_dispatch": ["layout_dispatch.hip", "row_io.hpp", "ep_device.hpp", "ep_internal.hpp"],
}


def kernel_source_hash(kernel=None):
    """Short hash of the sources of one kernel (all of csrc/ when kernel is
    None): identifies the code a counter summary was taken on."""
    import hashlib

    files = KERNEL_SOURCES[kernel] if kernel else sorted(os.listdir(CSRC))
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def common_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-ffp-contract=off",
        # packed fp32 instructions stay off (hipcc's host pass warns it does
        # not know the feature; the warning is harmless)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 8)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        results = list(pool.map(_compile, SOURCES))
    objs = [r[0] for r in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    build_c_abi_test()
    return LIB


C_TEST_SRC = os.path.join(ROOT, "tests", "c_abi_roundtrip.c")
C_TEST_BIN = os.path.join(BUILD, "c_abi_roundtrip")


def build_c_abi_test():
    """The C program that calls the library from C (tests/c_abi_roundtrip.c),
    compiled with gcc against the HIP runtime API and linked to libep.so."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(rocm, 'include')}",
           f"-I{INCLUDE}", C_TEST_SRC, "-o", C_TEST_BIN, f"-L{PKG}", "-lep", f"-L{os.path.join(rocm, 'lib')}",
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/..", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed on {C_TEST_SRC}:\n{res.stdout}\n{res.stderr}")
    return C_TEST_BIN


if __name__ == "__main__":
    print(build(verbose=True))
