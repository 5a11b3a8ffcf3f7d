"""The reciprocal form of the activation quantisation's division (CPU).

The router kernel quantises x per 128 columns by v / s with one scale per
group; it computes the quotients from one correctly rounded reciprocal and an
fma residual step instead of 32 IEEE divisions (the scale s >= 2^-64, finite;
other scales divide).  ``quotient_check.c`` compares the two for every bf16
group maximum and every bf16 value up to it: the e4m3 codes must be equal for
all of them (the GPU tests then check the codes bit-exactly against the
oracle on the configs' data).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.timeout(600)
def test_reciprocal_quotient_gives_the_ieee_codes(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "quotient_check"
    # -ffp-contract=off: the program's fmaf calls are the only fused operations
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", str(exe), os.path.join(HERE, "quotient_check.c"), "-lm"],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=580)
    print(r.stdout)
    fields = dict(zip(r.stdout.split()[0::2], map(int, r.stdout.split()[1::2])))
    assert fields["pairs"] > 900_000_000
    assert fields["fp32_differ_at_or_above_2^-10"] == 0
    assert fields["code_differ"] == 0
    assert r.returncode == 0
