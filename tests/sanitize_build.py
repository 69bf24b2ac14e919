"""Sanitizer builds for the CPU tests (test infrastructure; nothing here runs on
a GPU).

* the oracle (``oracle/ds_oracle.c``) built with clang under AddressSanitizer
  and UndefinedBehaviorSanitizer (single-threaded: no OpenMP);
* ``libds.so`` with the host code of ``csrc/api.hip`` (argument validation,
  workspace plan, dispatch, error paths) under the same sanitizers; its device
  code and the other translation units are the regular objects of the
  in-place build (``_build/``).

Both libraries need clang's sanitizer runtime loaded first; ``runtime()``
gives its path for LD_PRELOAD.
"""
from __future__ import annotations

import glob
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_decode_ds_amd")
LLVM = "/opt/rocm/llvm"
HIPCC = "/opt/rocm/bin/hipcc"

# host-only sanitizer flags; on a hipcc line each one follows -Xarch_host
_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
        "-fno-omit-frame-pointer"]


def runtime() -> str | None:
    """clang's shared ASan runtime (it carries the UBSan handlers too)."""
    hits = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def regular_objects() -> list[str]:
    """The in-place build's objects of every source but api.hip."""
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.o")))
    return [o for o in objs if os.path.basename(o) != "api.o"]


def build_oracle(out_dir: str) -> str:
    lib = os.path.join(out_dir, "liboracle_san.so")
    cmd = [os.path.join(LLVM, "bin", "clang"), "-O1", "-g", "-std=c11", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-shared", "-fPIC"] + _SAN + [
           os.path.join(ROOT, "oracle", "ds_oracle.c"), "-o", lib, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return lib


def build_libds(out_dir: str) -> str:
    api_o = os.path.join(out_dir, "api_san.o")
    host = []
    for f in _SAN:
        host += ["-Xarch_host", f]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-I" + os.path.join(ROOT, "include"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-fhip-fp32-correctly-rounded-divide-sqrt"] + host + [
           "-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    lib = os.path.join(out_dir, "libds_san.so")
    link = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-shared-libsan",
            "-Xarch_host", "-fsanitize=address,undefined", api_o] + regular_objects() + ["-o", lib]
    subprocess.run(link, check=True, capture_output=True, text=True)
    return lib
