"""The FP8 quantiser's fast scale and quotient against the definition, exhaustively on the CPU.

The pack kernel computes the block scale amax / 448 by a multiply with one FMA
correction, and divides by the scale through its reciprocal with one FMA
correction (blocks with amax >= 2^-64), ORing each x's sign bit into its code;
the method encodes the correctly rounded quotients.  ``quotient_check.c`` walks
every bf16 amax and every bf16 |x| <= amax, and counts the scales that differ
from the correctly rounded one and the pairs whose E4M3 codes differ: there
must be none.  Planted variants (no scale correction, no quotient correction,
no sign OR) must be caught, so the check has teeth."""

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
        return int(out[1]), int(out[3]), int(out[5])

    with ThreadPoolExecutor(max_workers=parts) as ex:
        res = list(ex.map(one, ranges))
    return tuple(sum(r[i] for r in res) for i in range(3))


QUOTIENT = "const float q1 = fmaf(fmaf(-q0, scale, x), r, q0);"
SCALE = "const float scale = fmaf(fmaf(-s0, 448.0f, amax), c, s0);"
SIGN = "return e4m3_code(fabsf(q1)) | (signbit(x) ? 0x80 : 0);"


def test_corrected_scale_and_quotient_give_the_same_e4m3_codes(tmp_path):
    checked, mismatches, scale_mismatches = _run(_build(tmp_path))
    # every positive finite bf16 amax >= 2^-64 paired with every bf16 0 <= x <= amax, and both zeros
    assert checked > 400_000_000
    assert mismatches == 0
    # every positive finite bf16 amax: the corrected product is the correctly rounded amax / 448
    assert scale_mismatches == 0


def test_check_catches_an_uncorrected_reciprocal(tmp_path):
    text = open(SRC).read()
    assert text.count(QUOTIENT) == 2
    text = text.replace(QUOTIENT, "const float q1 = q0;")
    _, mismatches, _ = _run(_build(tmp_path, text, "uncorrected"), lo=0x3F00, hi=0x4000, parts=4)
    assert mismatches > 0


def test_check_catches_an_uncorrected_scale(tmp_path):
    # the product with the rounded reciprocal of 448 alone is off by an ulp for about half of all amax
    text = open(SRC).read()
    assert text.count(SCALE) == 1
    text = text.replace(SCALE, "const float scale = s0;")
    _, _, scale_mismatches = _run(_build(tmp_path, text, "uncorrected_scale"), lo=0x3F00, hi=0x4000, parts=4)
    assert scale_mismatches > 0


def test_check_catches_the_lost_sign_of_minus_zero(tmp_path):
    # without x's sign ORed into the code, the correction turns -0 into +0: code 0x00 where the
    # quotient gives 0x80
    text = open(SRC).read()
    assert text.count(SIGN) == 1
    text = text.replace(SIGN, "return e4m3_code(fabsf(q1)) | (signbit(q1) ? 0x80 : 0);")
    _, mismatches, _ = _run(_build(tmp_path, text, "unsigned_zero"), lo=0x3F00, hi=0x3F10, parts=2)
    assert mismatches == 16          # -0 under each of the 16 amax values of the range, nothing else
