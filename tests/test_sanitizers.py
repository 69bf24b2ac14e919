"""The C ABI's host code (validation, workspace plan, dispatch, error paths of
csrc/api.hip) and the oracle run their CPU tests under AddressSanitizer and
UndefinedBehaviorSanitizer: test_abi.py, test_oracle.py and
test_oracle_calib.py in a child process with clang's sanitizer runtime
preloaded.  Any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import sanitize_build as sb  # noqa: E402


def test_abi_and_oracle_tests_under_asan_and_ubsan(tmp_path):
    rt = sb.runtime()
    if rt is None:
        pytest.skip("clang sanitizer runtime not installed")
    if not sb.regular_objects():
        pytest.skip("in-place build objects missing (run __graft_entry__.build())")
    libds = sb.build_libds(str(tmp_path))
    liboracle = sb.build_oracle(str(tmp_path))
    # reports go to files: pytest in the child holds its stderr while a test runs
    log = str(tmp_path / "san")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:log_path=" + log,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:log_path=" + log)
    r = subprocess.run([sys.executable, os.path.join(HERE, "san_runner.py"), libds, liboracle],
                       capture_output=True, text=True, timeout=900, env=env)
    out = r.stdout + r.stderr
    for f in sorted(tmp_path.glob("san*")):
        out += "\n" + f.read_text()
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout
    assert "loaded: %s %s" % (libds, liboracle) in r.stdout


def test_the_sanitizers_are_live(tmp_path):
    """A planted overflow in a call of the sanitized oracle (top-k indices
    written into too small an array) must be reported."""
    rt = sb.runtime()
    if rt is None:
        pytest.skip("clang sanitizer runtime not installed")
    liboracle = sb.build_oracle(str(tmp_path))
    code = ("import ctypes, numpy as np\n"
            "lib = ctypes.CDLL(%r)\n"
            "s = np.arange(5000, dtype=np.float64)\n"
            "out = np.zeros(4000, dtype=np.int32)\n"
            "lib.oracle_topk(ctypes.c_void_p(s.ctypes.data), 5000, 4096,"
            " ctypes.c_void_p(out.ctypes.data))\n" % liboracle)
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]
