"""Pins for the NF4 codebook (reading R1) against what the pages and the
mathematics fix: normal quantiles, normalised to [-1, 1], exact zero."""

import statistics
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import ndtr, ndtri

from oracle import nf4


def test_codebook_extremes_zero_and_order():
    c = nf4.codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert c[0] == -1.0 and c[15] == 1.0 and c[nf4.ZERO_CODE] == 0.0
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert int((c < 0).sum()) == 7 and int((c > 0).sum()) == 8


def test_codebook_two_independent_inverse_cdfs_agree_bitwise():
    a = nf4.codebook(statistics.NormalDist().inv_cdf)
    b = nf4.codebook(lambda p: float(ndtri(p)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_codebook_equal_probability_spacing():
    """Phi(c_j * Q(p_max)) is equally spaced on each side of zero, with steps
    (p_max - 1/2)/8 (positive side) and (p_max - 1/2)/7 (negative side)."""
    c = nf4.codebook().astype(np.float64)
    top = float(ndtri(nf4.P_MAX))
    pos = ndtr(c[c > 0] * top)            # ascending
    neg = ndtr(-c[c < 0] * top)           # descending magnitudes -> ascending p
    step_pos = (nf4.P_MAX - 0.5) / 8
    step_neg = (nf4.P_MAX - 0.5) / 7
    assert np.allclose(np.diff(pos), step_pos, atol=2e-7)
    assert np.allclose(np.diff(np.sort(neg)), step_neg, atol=2e-7)
    assert abs(pos[0] - (0.5 + step_pos)) < 2e-7 and abs(pos[-1] - nf4.P_MAX) < 2e-7


def test_codebook_is_symmetric_in_construction_not_values():
    """The extreme magnitudes match (+-1) but the interior does not: 7 negative
    and 8 positive quantile levels cannot mirror each other."""
    c = nf4.codebook()
    assert -c[0] == c[15]
    assert not np.allclose(-c[1:7][::-1], c[8:14])


def test_midpoints_are_exact_real_midpoints():
    c = nf4.codebook()
    m = nf4.midpoints()
    for j in range(15):
        exact = (Fraction(float(c[j])) + Fraction(float(c[j + 1]))) / 2
        assert Fraction(float(m[j])) == exact


@pytest.mark.parametrize("j", range(15))
def test_midpoint_fits_26_bits(j):
    """m_j has at most 26 significant bits, so absmax*m_j (24-bit absmax, 50
    bits in all) is exact in fp64 -- the basis of the exact nearest-code rule."""
    m = Fraction(float(nf4.midpoints()[j]))
    num = abs(m.numerator)
    while num and num % 2 == 0:
        num //= 2
    assert num.bit_length() <= 26
