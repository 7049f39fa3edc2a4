"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): cdl_oracle.c is rebuilt with -fsanitize=address,undefined and
-fno-sanitize-recover, and the oracle pin suites run against that build in a
child process, so that an out-of-bounds access, a signed overflow or an
invalid shift anywhere in the oracle fails the test instead of passing
silently.  The exhaustive fast-quotient check is left out (it runs the same
codec for a minute in its own test)."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

PIN_SUITES = ["test_oracle_layout.py", "test_oracle_dispatch_combine.py",
              "test_oracle_formats.py", "test_oracle_fp8_formats.py"]


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], stdout=subprocess.PIPE,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no libasan for gcc here")
    lib = str(tmp_path / "libcdl_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared",
                           "-ffp-contract=off", "-fno-fast-math",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", lib,
                           os.path.join(ROOT, "oracle", "cdl_oracle.c"), "-lm"])
    env = dict(os.environ)
    env.update({"CDL_ORACLE_LIB": lib, "LD_PRELOAD": asan,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", *[os.path.join(ROOT, "tests", f) for f in PIN_SUITES]],
                         cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True, timeout=900)
    tail = "\n".join(res.stdout.splitlines()[-30:])
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in res.stdout and "runtime error" not in res.stdout, tail
    assert " passed" in res.stdout, tail
