"""The fp8 kernels' division-free group arithmetic (scale, reciprocal and
quotient) gives the correctly rounded scale and reciprocal and the same
e4m3fn codes as x / s for every group it is applied to (exhaustive over bf16
inputs; CPU only, about a minute)."""
import os
import subprocess

from conftest import ROOT


def _cflags():
    flags = ["-O2", "-std=c99", "-ffp-contract=off"]
    try:
        with open("/proc/cpuinfo") as f:
            if " fma " in f.read():
                flags.append("-mfma")        # hardware fmaf: same result, faster
    except OSError:
        pass
    return flags


def test_fast_quotient_exhaustive(tmp_path):
    exe = str(tmp_path / "fast_quotient_check")
    subprocess.check_call(["gcc", *_cflags(), "-o", exe,
                           os.path.join(ROOT, "tests", "fast_quotient_check.c"),
                           os.path.join(ROOT, "oracle", "cdl_oracle.c"), "-lm"])
    res = subprocess.run([exe], stdout=subprocess.PIPE, text=True, timeout=600)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    assert "with amax >= 2^-96" in res.stdout
