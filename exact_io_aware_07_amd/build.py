"""Build libfa.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_07_amd.build

Every HIP source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into exact_io_aware_07_amd/libfa.so. The build always
recompiles; it needs no GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

ARCH = "gfx950"
# Packed fp32 VALU instructions are turned off: only scalar fp32 VALU forms
# are generated for every kernel.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; set HIPCC or install ROCm")
    return cand


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device feature above and says so;
    # that line is expected and dropped.
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-sanitized variant (AddressSanitizer and UndefinedBehaviorSanitizer on
# the host code only: argument validation and the block-sparse planner; the
# device code is built as usual). For tests on the CPU; never installed.
SAN_DIR = os.path.join(BUILD, "host_sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libfa_host_sanitized.so")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
                 "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it also holds
    the UndefinedBehaviorSanitizer handlers)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("amdclang") or "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise RuntimeError("the compiler's shared AddressSanitizer runtime was not found")
    return out


def build_host_sanitized() -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sources()

    def one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *HOST_SANITIZE, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    rt = asan_runtime()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", SAN_LIB, *objs, rt,
           f"-Wl,-rpath,{os.path.dirname(rt)}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    if sys.argv[1:] == ["--host-sanitized"]:
        print(build_host_sanitized())
    else:
        print(build(verbose=True))
