"""The e4m3 quantisers compute v / s without a division per value: the product
v * fp32(1 / s) corrected once by the exact FMA remainder.  quotient_check.c
checks on the CPU that this reproduces the IEEE fp32 quotient wherever the
e4m3 code depends on it (blocks with s >= 2^-90; the kernels divide for
smaller scales).  The default cases below cover, exhaustively, every bf16 pair
for block maxima near the 2^-90 scale limit, around 1 and at the top of the
range, and 2e6 random fp32 block maxima with values on and next to the
rounding ties of the codes; `quotient_check bf16 -82 127` covers every bf16
pair (1.0e9 pairs, about 35 s).  The uncorrected product must fail the same check."""
import os
import shutil
import subprocess

import pytest

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quotient_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("needs a C compiler")
    exe = str(tmp_path_factory.mktemp("quotient") / "quotient_check")
    subprocess.run([cc, "-O2", "-std=c11", "-ffp-contract=off", SRC, "-o", exe, "-lm"],
                   check=True, capture_output=True, text=True)
    return exe


def run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=300)
    n, m = (int(x) for x in r.stdout.split()[-3::2])
    return r.returncode, n, m, r.stdout


@pytest.mark.parametrize("args", [("bf16", -82, -78), ("bf16", -4, 4), ("bf16", 123, 127),
                                  ("fp32", 2_000_000, 1)],
                         ids=["bf16-near-limit", "bf16-unit", "bf16-top", "fp32-random-ties"])
def test_corrected_product_is_the_ieee_quotient(checker, args):
    rc, n, m, out = run(checker, *args)
    assert rc == 0 and m == 0, out
    assert n > 5_000_000


def test_uncorrected_product_fails_the_check(checker):
    rc, n, m, out = run(checker, "fp32", 100_000, 1, "plain")
    assert rc == 1 and m > 0.01 * n, out
