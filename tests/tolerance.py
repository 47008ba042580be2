"""Tolerance for fp32 results that are binary64 sums of exact terms rounded
once to binary32 (the combine backward's weight and bias gradients).

A reference computed in binary64 in another order differs from the exact sum
by at most n * 2^-52 * sum|terms| (n terms, standard recursive-summation
bound with n * u < 1); rounding the GPU's binary64 sum to binary32 adds at
most half an ulp, 2^-24 |value|.  So |gpu - ref| <= 2^-24 |ref| +
n 2^-52 sum|terms| (the 2^-24 term also absorbs the tiny difference between
|gpu| and |ref|)."""
import numpy as np


def sum_bound(ref, mag, n):
    return 2.0 ** -24 * np.abs(ref) + n * 2.0 ** -52 * mag + 1e-300


def check_sum(got, ref, mag, n):
    """Assert the binary32 results `got` are within the bound of the
    binary64 references `ref` (terms' magnitudes summed in `mag`)."""
    excess = np.abs(np.asarray(got, np.float64) - ref) - sum_bound(ref, mag, n)
    assert np.all(excess <= 0), float(np.max(excess))
