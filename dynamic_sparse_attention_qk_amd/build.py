"""Builds libdsa.so (all HIP sources, gfx950) in-tree with hipcc, and two variants of it that differ only in
api.hip (the C ABI's host layer; every other object is shared):
  libdsa_debug.so  compiled with DSA_DEBUG: the attention calls check their kept-block lists and reverse
                   index on the device first and return DSA_ERR_BAD_LIST on a malformed one;
  libdsa_san.so    the host code of api.hip under AddressSanitizer and UndefinedBehaviorSanitizer (device code
                   unchanged); load it with the sanitizer runtime preloaded (tests/test_sanitized_abi.py).
The binding loads a variant when DSA_LIBRARY names it.

Usage: python -m dynamic_sparse_attention_qk_amd.build [--verbose] [--release-only]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsa.so")
SOURCES = ["api.hip", "predict.hip", "predict_train.hip", "predict_pooled.hip", "select.hip", "attn_fwd.hip",
           "attn_bwd.hip", "validate.hip"]
DEBUG_LIB = os.path.join(PKG, "libdsa_debug.so")
SAN_LIB = os.path.join(PKG, "libdsa_san.so")
# host-only sanitizer flags: each -fsanitize applies to the host compilation alone (-Xarch_host)
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def _link(objs, lib, verbose, extra=()):
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs], verbose)
    os.replace(tmp, lib)


def build(verbose: bool = False, jobs: int = 5, variants: bool = True) -> str:
    """Compile every HIP source and link libdsa.so (and, with variants, libdsa_debug.so and libdsa_san.so);
    returns the path of libdsa.so."""
    os.makedirs(OBJ, exist_ok=True)
    jobs_list = [(src, os.path.join(OBJ, src.replace(".hip", ".o")), FLAGS) for src in SOURCES]
    if variants:
        jobs_list += [("api.hip", os.path.join(OBJ, "api_debug.o"), FLAGS + ["-DDSA_DEBUG"]),
                      ("api.hip", os.path.join(OBJ, "api_san.o"), [f for f in FLAGS if f != "-O3"] + ["-O1"] +
                       SAN_FLAGS)]

    def compile_one(job):
        src, out, flags = job
        _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", out], verbose)
        return out

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(compile_one, jobs_list))
    objs = outs[:len(SOURCES)]
    _link(objs, LIB, verbose)
    if variants:
        rest = objs[1:]  # every object but api.o
        _link([outs[len(SOURCES)]] + rest, DEBUG_LIB, verbose)
        _link([outs[len(SOURCES) + 1]] + rest, SAN_LIB, verbose,
              extra=["-fsanitize=address,undefined", "-shared-libsan"])
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, variants="--release-only" not in sys.argv))
