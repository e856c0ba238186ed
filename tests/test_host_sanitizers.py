"""The library's host code under AddressSanitizer + UndefinedBehaviorSanitizer
(CPU only): argument validation and workspace layout, the Algorithm 1
planner and the KV-exchange map builders are integer host code reached
through ctypes.  The host-sanitized build (`python -m
document_masked_attention_amd.build --host-asan`) is loaded in a child Python
with the sanitizer runtime preloaded, and the host-logic test files run there;
any sanitizer report fails the run (UBSan does not recover)."""
import os
import subprocess
import sys

import pytest

from document_masked_attention_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_abi_cpu.py", "tests/test_plan_host.py", "tests/test_exchange_host.py"]


def _stale() -> bool:
    if not os.path.exists(build.ASAN_LIB):
        return True
    t = os.path.getmtime(build.ASAN_LIB)
    srcs = [os.path.join(build.CSRC, s) for s in os.listdir(build.CSRC)] + [os.path.join(build.INCLUDE, "docmask.h")]
    return any(os.path.getmtime(p) > t for p in srcs)


@pytest.fixture(scope="module")
def asan_lib():
    if _stale():
        build.build_host_asan()
    return build.ASAN_LIB


def test_sanitized_build_is_instrumented(asan_lib):
    r = subprocess.run(["nm", "-D", "--undefined-only", asan_lib], capture_output=True, text=True, check=True)
    assert "__asan_report_load" in r.stdout or "__asan_load" in r.stdout
    assert "__ubsan_handle_" in r.stdout


def test_host_code_clean_under_asan_and_ubsan(asan_lib):
    env = dict(os.environ)
    env.update({
        "DOCMASK_LIBRARY": asan_lib,
        "LD_PRELOAD": build.host_asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    code = ("import sys, pytest\n"
            "from document_masked_attention_amd import api\n"
            "api.lib()\n"
            "maps = open('/proc/self/maps').read()\n"
            "assert 'libdocmask_asan.so' in maps and 'libclang_rt.asan' in maps, 'sanitized library not loaded'\n"
            f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', *{HOST_TESTS!r}]))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
