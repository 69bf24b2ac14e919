"""Runs the CPU tests of the C ABI and of the oracle against sanitizer builds
(test infrastructure): san_runner.py LIBDS_SAN LIBORACLE_SAN.  Start it with
clang's ASan runtime in LD_PRELOAD (sanitize_build.runtime())."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import pytest  # noqa: E402

import oracle  # noqa: E402
import sparse_attention_decode_ds_amd as ds  # noqa: E402

ds.LIB_PATH = os.path.abspath(sys.argv[1])
oracle._LIB = os.path.abspath(sys.argv[2])
rc = pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                  os.path.join(ROOT, "tests", "test_abi.py"),
                  os.path.join(ROOT, "tests", "test_oracle.py"),
                  os.path.join(ROOT, "tests", "test_oracle_calib.py")])
# the libraries the tests actually ran against
print("loaded:", ds.load()._name, oracle._load()._name, flush=True)
sys.exit(rc)
