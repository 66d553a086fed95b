"""The activation-quantisation kernel and the decode kernel's in-prologue
quantiser form v/s from the reciprocal of the scale and one fma correction
instead of a division.  This
checks, exhaustively on the host, that the codes it gives equal those of the
IEEE division the activation quantiser is defined with (code =
clamp(rint(v / s), -7, 7), s = amax / 7 in fp32), for every fp16 amax and
every fp16 value within it: the quotient itself is identical up to the sign
of a zero quotient.  The C program restates the kernel's three operations;
the library is not involved."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_quotient_gives_identical_codes(tmp_path):
    exe = tmp_path / "quotient_identity"
    subprocess.run(["gcc", "-O2", "-mfma", "-o", str(exe), os.path.join(HERE, "csrc", "quotient_identity.c"),
                    "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    fields = out.stdout.split()
    got = dict(zip(fields[0::2], map(int, fields[1::2])))
    # amax bit patterns 0 .. 0x7C00 (+inf), each with 2 * (its index + 1) values v
    n = 0x7C01
    assert got["pairs"] == n * (n + 1)
    assert got["code_mismatch"] == 0
    assert got["nonzero_mismatch"] == 0
    assert out.returncode == 0
