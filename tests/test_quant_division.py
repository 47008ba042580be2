"""The FP8 quantiser divides finite blocks through one correctly rounded
reciprocal of the scale and one fused multiply-add correction (Markstein's
scheme) instead of a division per value, and divides by a UE8M0 power of two
with one multiplication.  Per-block scales follow DeepEP notes ch.7, s7.1.
The whole input domain is small enough to enumerate: every finite bf16 block
maximum fixes the scale, and every bf16 value no larger in magnitude is a
possible dividend (about 1.07e9 pairs).  This compiles a plain C check with
gcc and requires every pair to give the correctly rounded quotient wherever
the E4M3 code can depend on it.  CPU only."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_reciprocal_division_is_correctly_rounded_on_the_whole_domain(tmp_path):
    exe = str(tmp_path / "quant_division_check")
    cc = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          os.path.join(HERE, "quant_division_check.c"), "-o", exe, "-lm"]
    if subprocess.run(cc + ["-fopenmp"], capture_output=True).returncode != 0:
        subprocess.run(cc, check=True, capture_output=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600, check=True)
    pairs, bad_rcp, bad_pow2 = map(int, out.stdout.split())
    # sum over amax patterns a of 2 (a + 1), a = 0 .. 0x7F7F
    n = 0x7F80
    assert pairs == n * (n + 1)
    assert bad_rcp == 0
    assert bad_pow2 == 0
