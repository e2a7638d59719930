"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU.

libdsa_san.so is the library with api.hip's host code compiled with -fsanitize=address,undefined (any
undefined behaviour aborts; device code unchanged).  tests/test_abi.py -- every argument check, status and
workspace size the host layer computes -- runs against it in a child process that has the sanitizer
runtime preloaded (python itself is not instrumented), and the debug build must export the same symbols.
"""
import glob
import os
import subprocess
import sys

import pytest

import dynamic_sparse_attention_qk_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dynamic_sparse_attention_qk_amd")


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_suite_under_asan_ubsan():
    lib = os.path.join(PKG, "libdsa_san.so")
    rt = _asan_runtime()
    if not os.path.exists(lib) or rt is None:
        pytest.skip("libdsa_san.so or the ASan runtime is missing (python -m dynamic_sparse_attention_qk_amd.build)")
    env = dict(os.environ)
    env.update(DSA_LIBRARY="libdsa_san.so", LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    probe = ("import dynamic_sparse_attention_qk_amd as d; d.library(); "
             "maps = open('/proc/self/maps').read(); "
             "assert 'libdsa_san.so' in maps and 'libclang_rt.asan' in maps, 'sanitized library not loaded'; "
             "print('loaded', d.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail


def test_debug_build_exports_the_same_calls():
    path = os.path.join(PKG, "libdsa_debug.so")
    if not os.path.exists(path):
        pytest.skip("libdsa_debug.so is missing (python -m dynamic_sparse_attention_qk_amd.build)")
    lib = dsa.load_library(path)
    for name in dsa.EXPORTED:
        assert hasattr(lib, name), name
    assert lib.dsa_status_string(-9) != dsa.library().dsa_status_string(5)  # -9 has its own text
