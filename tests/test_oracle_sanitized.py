"""The oracle's C source under the host sanitizers.

oracle.c is rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only; every UB report aborts) into a temporary library, and
every pin runs against that build in a child process with the ASan runtime
loaded first.  An out-of-bounds access, a use after free, a signed overflow,
a misaligned load or an invalid shift in the oracle then fails this test
even where it would not change a pinned value.  Leak checking is off: the
child is a Python interpreter, whose own allocations would be reported.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc has no ASan runtime here")
def test_pins_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", str(lib), SRC, "-lm"], check=True)
    env = dict(os.environ)
    preload = [_runtime("libasan.so")] + ([env["LD_PRELOAD"]] if env.get("LD_PRELOAD") else [])
    env["LD_PRELOAD"] = ":".join(preload)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), str(lib)],
                         capture_output=True, text=True, timeout=600, cwd=ROOT, env=env)
    assert res.returncode == 0, f"pins under the sanitizers failed:\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
