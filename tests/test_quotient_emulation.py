"""The kernels' division-free quotient x / s, emulated on the CPU, against IEEE binary32 division.

The GPU decides every code from clamp(rint(x / s + zero)) (page "LLM 量化方法原理与实现详解", §2.2: the
printed quantizers round x / scale (+ zero_point) in the tensor's precision), with x / s formed by a
reciprocal and Markstein's correction instead of a division per element.  ``quotient_check.c`` emulates
that formula step by step with the C library's correctly rounded fmaf and counts disagreements with the
division: over every mantissa of the scaled scale s' in [1, 2) with quotients at and next to the ties of
rint, and over random (x, s) across the whole binary32 range through the full path (scaling, clamp).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path_factory.mktemp("qc") / "quotient_check")
    subprocess.run([cc, "-O2", "-fopenmp", "-ffp-contract=off", os.path.join(HERE, "quotient_check.c"), "-o", exe,
                    "-lm"], check=True)
    return exe


def _run(exe, *args):
    out = subprocess.run([exe, *map(str, args)], check=True, capture_output=True, text=True, timeout=600).stdout
    bad_q, bad_code, checked = map(int, out.split())
    return bad_q, bad_code, checked


def test_quotient_equals_division_every_scale_mantissa(checker):
    bad_q, bad_code, checked = _run(checker, 1, 2_000_000)
    assert checked > 1_400_000_000  # 2^23 mantissas x 175 quotients, and the random pairs
    assert bad_q == 0 and bad_code == 0, (bad_q, bad_code)
