"""Build libmoe.so (HIP, gfx950) in-tree with hipcc."""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


LIB_DEBUG = os.path.join(PKG, "libmoe_debug.so")
# The debug build: host-side checks of the permutation arrays before every
# launch that indexes with them (moe_check_permutation).
DEBUG_FLAGS = ["-DMOE_HOST_BOUNDS_CHECK", "-O2", "-g"]
# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (the GPU
# code is built as usual); loaded by a sanitized host program only.
HOST_SANITIZE_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                       "-Xarch_host -fno-sanitize-recover=all "
                       "-Xarch_host -fno-omit-frame-pointer -g").split()


def sources():
    csrc = os.path.join(PKG, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.cpp")))


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_debug(verbose: bool = False) -> str:
    return build(verbose, LIB_DEBUG, DEBUG_FLAGS)


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    return build(verbose, out, HOST_SANITIZE_FLAGS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--debug" in sys.argv:
        print(build_debug(verbose="-v" in sys.argv))
