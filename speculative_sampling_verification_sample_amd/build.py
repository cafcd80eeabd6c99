"""Compile the HIP library (libspecverify.so) in-tree for gfx950 with hipcc."""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
# Host-sanitized variant for the CPU-side checks of the C ABI: the host code
# built with AddressSanitizer and UndefinedBehaviorSanitizer (device code
# unchanged); it is loaded with the ASan runtime preloaded.
LIB_HOSTSAN = os.path.join(PKG, "libspecverify_hostsan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # identical rounding in every kernel: no implicit fma contraction
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


HOSTSAN_FLAGS = [
    "-O1", "-g",
    "-Xarch_host", "-fsanitize=address,undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def build(verbose: bool = False, hostsan: bool = False) -> str:
    """Compile csrc/specverify.hip into libspecverify.so (hostsan: the
    host-sanitized libspecverify_hostsan.so); returns the path."""
    src = os.path.join(CSRC, "specverify.hip")
    out = LIB_HOSTSAN if hostsan else LIB
    tmp = out + ".tmp"
    flags = [f for f in FLAGS if f != "-O3"] + HOSTSAN_FLAGS if hostsan else FLAGS
    cmd = [HIPCC, *flags, f"-I{INCLUDE}", f"-I{CSRC}", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime ('' if it is not there)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    try:
        r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    except OSError:
        return ""
    path = r.stdout.strip()
    if os.path.isabs(path) and os.path.exists(path):
        return path
    res = subprocess.run([clang, "-print-resource-dir"], capture_output=True, text=True).stdout.strip()
    path = os.path.join(res, "lib", "linux", "libclang_rt.asan-x86_64.so")
    return path if os.path.exists(path) else ""


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, hostsan="--hostsan" in sys.argv))
