"""Build libdocmask.so (HIP, gfx950) in-tree with hipcc.

    python -m document_masked_attention_amd.build              # the library
    python -m document_masked_attention_amd.build --host-asan  # + a host-sanitized copy

The host-sanitized copy (_build/asan/libdocmask_asan.so) instruments only the
host code (argument validation, workspace layout, the planner and the
exchange map builders) with AddressSanitizer and UndefinedBehaviorSanitizer;
its GPU code is built exactly as in the library.  Load it by setting
DOCMASK_LIBRARY to its path and preloading the sanitizer runtime
(host_asan_runtime()); the CPU tests do this in a subprocess.
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
LIB = os.path.join(PKG, "libdocmask.so")
SOURCES = ["abi.hip", "sched.hip", "fwd.hip", "bwd.hip", "merge.hip", "timing.hip", "exchange.hip", "plan.hip",
           "probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
    # packed fp32 VALU instructions stay off (ordinary float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# sanitizers for the host pass only (each -fsanitize= right after -Xarch_host)
HOST_SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
]
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libdocmask_asan.so")


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


BWD_ASM = os.path.join(BUILD, "bwd-gfx950.s")


def check_inline_mfma_wait_states(verbose: bool = False) -> int:
    """Generate the gfx950 assembly of bwd.hip and check the dK/dV kernel's
    inline-assembly MFMAs (see isa_check); raises on any violation.  Returns
    the number of MFMAs checked."""
    from . import isa_check
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "bwd.hip"), "-o", BWD_ASM]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for bwd.hip:\n{r.stderr}")
    asm = open(BWD_ASM).read()
    syms = isa_check.kernel_symbols(asm)
    if not syms:
        raise RuntimeError("no dK/dV kernel found in the generated assembly")
    total, bad = 0, []
    for sym in syms:
        n, v = isa_check.check(asm, sym)
        total += n
        bad += v
    if bad:
        raise RuntimeError("inline MFMA results touched inside the wait-state window:\n" + "\n".join(bad))
    if verbose:
        print(f"wait states of {total} inline MFMAs checked in {len(syms)} dK/dV kernels")
    return total


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES) + 1) as ex:
        chk = ex.submit(check_inline_mfma_wait_states, verbose)
        objs = list(ex.map(_compile, SOURCES))
        chk.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def host_asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (it also holds
    the UndefinedBehaviorSanitizer handlers)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's compiler was not found")
    return path


def build_host_asan(verbose: bool = False) -> str:
    """The library with host-side ASan + UBSan (see the module docstring)."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, ASAN_DIR, HOST_SANITIZE_FLAGS), SOURCES))
    tmp = ASAN_LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print("built", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    if "--host-asan" in sys.argv[1:]:
        build_host_asan(verbose=True)
    sys.exit(0)
