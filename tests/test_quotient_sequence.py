"""The bulk prefill quantizer's quotient sequence equals correctly rounded
division on every input it can meet.

quant_append_bulk_kernel divides a row's values by the row's scale with one
correctly rounded reciprocal and three operations per value (Markstein's
correction step) instead of a correctly rounded division per value. The
codes must stay bit-identical to the plain definition (the "KV Cache
optimization techniques" tutorial, section 1.2: code = round(x / scale) with
scale = max-abs / 127, or / 7 for INT4), so this test checks the identity
exhaustively on the host: every fp16 value x against every fp16 max-abs a
with |x| <= a, at both code widths, about 2e9 pairs in C. The GPU kernel's
own codes are checked against the oracle by the parity tests.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_quotient_sequence_exhaustive(tmp_path):
    exe = str(tmp_path / "quotient_sequence_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "quotient_sequence_check.c"),
                    "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    lines = [l for l in r.stdout.splitlines() if l.startswith("qmax")]
    assert len(lines) == 2 and all(l.endswith(" 0 mismatches") for l in lines), r.stdout
