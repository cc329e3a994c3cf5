"""The FP8 quantiser's fast quotient against the definition, exhaustively on the CPU.

The pack kernel divides by the block scale through its reciprocal with one FMA
correction (blocks with amax >= 2^-64); the method encodes the correctly rounded
quotient.  ``quotient_check.c`` walks every bf16 amax and every bf16 |x| <= amax
and counts pairs whose E4M3 codes differ: there must be none.  A planted
variant without the correction step must be caught, so the check has teeth."""

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "quotient_check.c")


def _build(tmp_path, src_text=None, name="quotient_check"):
    src = SRC
    if src_text is not None:
        src = str(tmp_path / f"{name}.c")
        with open(src, "w") as f:
            f.write(src_text)
    exe = str(tmp_path / name)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
    return exe


def _run(exe, lo=0, hi=0x7F80, parts=8):
    step = (hi - lo + parts - 1) // parts
    ranges = [(a, min(hi, a + step)) for a in range(lo, hi, step)]

    def one(r):
        out = subprocess.run([exe, str(r[0]), str(r[1])], check=True, capture_output=True, text=True).stdout.split()
        return int(out[1]), int(out[3])

    with ThreadPoolExecutor(max_workers=parts) as ex:
        res = list(ex.map(one, ranges))
    return sum(c for c, _ in res), sum(m for _, m in res)


def test_corrected_reciprocal_quotient_gives_the_same_e4m3_codes(tmp_path):
    checked, mismatches = _run(_build(tmp_path))
    # every positive finite bf16 amax >= 2^-64 paired with every bf16 0 <= x <= amax
    assert checked > 400_000_000
    assert mismatches == 0


def test_check_catches_an_uncorrected_reciprocal(tmp_path):
    text = open(SRC).read().replace("const float q1 = copysignf(fmaf(fmaf(-q0, scale, x), r, q0), x);",
                                    "const float q1 = q0;")
    assert "q1 = q0;" in text
    checked, mismatches = _run(_build(tmp_path, text, "uncorrected"), lo=0x3F00, hi=0x4000, parts=4)
    assert mismatches > 0


def test_check_catches_the_lost_sign_of_minus_zero(tmp_path):
    # without the sign copy the correction turns -0 into +0: code 0x00 where the quotient gives 0x80
    text = open(SRC).read().replace("const float q1 = copysignf(fmaf(fmaf(-q0, scale, x), r, q0), x);",
                                    "const float q1 = fmaf(fmaf(-q0, scale, x), r, q0);")
    assert text.count("const float q1 = fmaf(") == 2
    checked, mismatches = _run(_build(tmp_path, text, "unsigned_zero"), lo=0x3F00, hi=0x3F10, parts=2)
    assert mismatches == 16          # -0 under each of the 16 amax values of the range, nothing else
