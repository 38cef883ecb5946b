"""The C-ABI tests under AddressSanitizer (host code of libmlap.so) and the oracle's pins
under UndefinedBehaviorSanitizer, each in a child process of its own (tests/sanitize.py)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_under_asan_and_oracle_pins_under_ubsan():
    r = subprocess.run([sys.executable, os.path.join(HERE, "sanitize.py")], stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:]
    assert r.stdout.count(" passed") == 2 and " failed" not in r.stdout, r.stdout[-4000:]
    assert "sanitizer runs: ok" in r.stdout
