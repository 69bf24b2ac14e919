"""Build libds.so (HIP, gfx950) in place with hipcc: one object per source,
compiled in parallel, then one shared-library link."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libds.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
HEADERS = sorted(glob.glob(os.path.join(HERE, "csrc", "*.h"))) + [os.path.join(ROOT, "include", "ds.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"),
    # packed fp32 instructions stay off; division and sqrt stay IEEE-exact
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
]


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n or (os.cpu_count() or 1), 16, len(SOURCES)))


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = ".tmp%d" % os.getpid()
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in SOURCES]

    def compile_one(src_obj):
        src, obj = src_obj
        cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj + tag]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, obj, r

    with ThreadPoolExecutor(_jobs()) as ex:
        results = list(ex.map(compile_one, zip(SOURCES, objs)))
    failed = [(src, r) for src, _, r in results if r.returncode != 0]
    for src, _, r in results:
        if verbose and r.stderr:
            sys.stderr.write(r.stderr)
    if failed:
        for src, r in failed:
            sys.stderr.write("hipcc failed on %s:\n%s\n" % (src, r.stderr))
        raise subprocess.CalledProcessError(failed[0][1].returncode, HIPCC)
    for _, obj, _ in results:
        os.replace(obj + tag, obj)
    tmp = LIB + tag
    cmd = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
