"""Build libsgmv.so, the HIP library behind the SGMV C ABI, for gfx950.

    python -m segmented_gather_gemv_sgmv_amd.build

compiles ``csrc/sgmv_api.hip`` (which includes the kernel headers) with
hipcc into ``libsgmv.so`` next to this file.  Cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libsgmv.so")
SOURCES = [os.path.join(CSRC, "sgmv_api.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Keep the compiler from forming packed fp32 instructions (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(output: str = LIBRARY, extra_flags=(), verbose: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


# The same library with its HOST code under AddressSanitizer, for the CPU
# tests of the C ABI's argument checks (no kernel runs there, so the device
# code is compiled unoptimised, which keeps the build short).  Loaded with
# the sanitizer runtime preloaded (ASAN_RUNTIME) and SGMV_LIBRARY pointing
# at it; never used on a GPU.
ASAN_LIBRARY = os.path.join(PKG, "libsgmv_asan.so")
ASAN_FLAGS = [
    f"--offload-arch={ARCH}",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-O1",
    "-Xarch_host", "-g",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-shared-libasan",
    "-Xarch_device", "-O0",
    "-w",
]


def asan_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime in the ROCm toolchain."""
    import glob
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(rocm, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under " + rocm)
    return hits[-1]


def sources_mtime() -> float:
    paths = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    paths += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    return max(os.path.getmtime(p) for p in paths)


def build_asan(output: str = ASAN_LIBRARY, verbose: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = [hipcc(), *ASAN_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def build_all(verbose: bool = False) -> None:
    """The library and its host-sanitizer variant, compiled side by side."""
    cmd_main = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", LIBRARY + ".tmp", *SOURCES]
    cmd_asan = [hipcc(), *ASAN_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", ASAN_LIBRARY + ".tmp",
                *SOURCES]
    procs = []
    for cmd in (cmd_main, cmd_asan):
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
    codes = [p.wait() for p in procs]
    if any(codes):
        raise subprocess.CalledProcessError(max(codes), "hipcc")
    os.replace(LIBRARY + ".tmp", LIBRARY)
    os.replace(ASAN_LIBRARY + ".tmp", ASAN_LIBRARY)


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan(verbose="-v" in sys.argv))
    elif "--all" in sys.argv:
        build_all(verbose="-v" in sys.argv)
    else:
        print(build(verbose="-v" in sys.argv))
