"""The staged parity check under the bounds-checked debug build (libmlap_debug.so, compiled with
MLAP_DEBUG), at ragged batch sizes on every tile shape, in a child process of its own
(tests/debug_parity.py): every case must match the oracle and leave no failed bounds check."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_debug_build_parity_and_bounds_checks():
    lib = os.path.join(ROOT, "mla_prolog_amd", "libmlap_debug.so")
    assert os.path.exists(lib), "the debug build is missing (run __graft_entry__.build())"
    env = dict(os.environ, MLAP_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "debug_parity.py")], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    print(r.stdout[-6000:], flush=True)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "every bounds check held" in r.stdout
