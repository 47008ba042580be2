"""The binary32-of-binary64 tolerance accepts what it must and rejects a
result one binary32 ulp off (CPU only)."""
import numpy as np
import pytest

from tests.tolerance import check_sum


def _case(seed, n=7168):
    rng = np.random.default_rng(seed)
    terms = rng.standard_normal(n) * rng.standard_normal(n)
    return terms, float(np.sum(terms)), float(np.sum(np.abs(terms)))


def test_accepts_rounded_sums_in_any_order():
    for seed in range(20):
        terms, ref, mag = _case(seed)
        other = float(np.sum(np.random.default_rng(seed + 99).permutation(terms)))
        check_sum(np.float32(other), np.array(ref), np.array(mag), terms.size)
        check_sum(np.float32(ref), np.array(ref), np.array(mag), terms.size)


def test_rejects_one_ulp_off():
    for seed in range(20):
        terms, ref, mag = _case(seed)
        r32 = np.float32(ref)
        for off in (np.nextafter(r32, np.float32(np.inf)), np.nextafter(r32, np.float32(-np.inf))):
            # one of the two neighbours may still be within half an ulp of ref
            # plus the reordering term; two ulps away never is
            far = np.nextafter(off, np.float32(np.inf) if off > r32 else np.float32(-np.inf))
            with pytest.raises(AssertionError):
                check_sum(far, np.array(ref), np.array(mag), terms.size)


def test_rejects_a_dropped_term():
    terms, ref, mag = _case(3)
    got = np.float32(ref - terms[np.argmax(np.abs(terms))])
    with pytest.raises(AssertionError):
        check_sum(got, np.array(ref), np.array(mag), terms.size)
