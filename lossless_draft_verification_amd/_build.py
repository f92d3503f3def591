"""Build the HIP library in-tree: libspecverify.so for gfx950 (MI355X)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "specverify.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")

# -ffp-contract=off: the arithmetic is exactly what the source writes (every
# fused multiply-add is an explicit fmaf).  Packed fp32 instructions are
# switched off for the device code.  The atomic optimizer is off: it turns
# the scan's one-lane append to the residual work list into a wave-combined
# atomic whose result is waited for at once, which puts the atomic's round
# trip on the scan's critical path (without it the wait falls after the
# draw plan is written).
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


# Host-code sanitizers (CPU checks only; the device code is built as usual):
# every -fsanitize= applies to the host pass alone.
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]
SAN_LIB = os.path.join(PKG, "libspecverify_san.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that a process loading the
    sanitized library must preload."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.check_output([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    if os.path.isabs(out) and os.path.exists(out):
        return out
    rt = subprocess.check_output([clang, "-print-runtime-dir"], text=True).strip()
    return os.path.join(rt, "libclang_rt.asan-x86_64.so")


def build(verbose: bool = False, sanitize: bool = False, path: str = "") -> str:
    """Compile the library (gfx950).  With `sanitize`, a build whose host code
    carries AddressSanitizer and UndefinedBehaviorSanitizer (-O1 -g), written
    to libspecverify_san.so (or `path`); load it with asan_runtime() preloaded
    and SPEC_LIBRARY pointing at it."""
    out = path or (SAN_LIB if sanitize else LIB)
    tmp = out + ".tmp"
    flags = list(HIPCC_FLAGS)
    if sanitize:
        flags = [f for f in flags if f != "-O3"] + ["-O1", "-g"] + SANITIZE_FLAGS
    cmd = [hipcc(), *flags, "-I", INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_abi_caller.c")
C_CALLER = os.path.join(ROOT, "tests", "_bin", "c_abi_caller")


def rocm_root() -> str:
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    return root if os.path.isdir(os.path.join(root, "include", "hip")) else "/opt/rocm"


def build_c_caller(verbose: bool = False) -> str:
    """Compile tests/c_abi_caller.c, a plain C program that calls the
    library through include/specverify.h and the HIP runtime's C API (gcc,
    no HIP compiler), against the in-tree libspecverify.so."""
    rocm = rocm_root()
    os.makedirs(os.path.dirname(C_CALLER), exist_ok=True)
    tmp = C_CALLER + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", INCLUDE, C_CALLER_SRC, "-o", tmp,
           "-L", PKG, "-lspecverify", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../lossless_draft_verification_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, C_CALLER)
    return C_CALLER


if __name__ == "__main__":
    print(build(verbose=True))
