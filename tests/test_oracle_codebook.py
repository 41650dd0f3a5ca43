"""Pins of the oracle's NF4 codebook against things other than itself.

The codebook definition ("qlora" entry, tonho.wtf, section "como funciona"):
standard-normal quantiles, normalised to [-1, 1] by the largest, equal
expected count per bin, asymmetric with an exact zero.
"""

import mpmath
import numpy as np
import pytest
from scipy.special import ndtr, ndtri

import oracle
from oracle.codebook import _DELTA

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def test_structure():
    cb = oracle.nf4_codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert cb[0] == -1.0 and cb[15] == 1.0
    assert cb[7] == 0.0 and not np.signbit(cb[7])  # exact zero
    assert np.all(np.diff(cb) > 0)
    assert (cb < 0).sum() == 7 and (cb > 0).sum() == 8  # asymmetric
    assert np.all(np.abs(cb) <= 1.0)


def _levels_mpmath():
    mpmath.mp.dps = 60
    d = mpmath.mpf(1) - (mpmath.mpf(1) / 32 + mpmath.mpf(1) / 30) / 2

    def inv_phi(p):
        return mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)

    top = inv_phi(d)
    pos = [inv_phi(mpmath.mpf(1) / 2 + j * (d - mpmath.mpf(1) / 2) / 8) / top for j in range(1, 9)]
    neg = [-inv_phi(mpmath.mpf(1) / 2 + j * (d - mpmath.mpf(1) / 2) / 7) / top for j in range(1, 8)]
    return sorted(neg + [mpmath.mpf(0)] + pos)


def test_bits_match_60_digit_evaluation():
    """An independent 60-digit evaluation (mpmath erfinv) rounds to the same fp32 bits."""
    cb = oracle.nf4_codebook()
    lv = _levels_mpmath()
    for k, v in enumerate(lv):
        f32 = np.float32(float(v))
        assert f32.view(np.uint32) == cb[k].view(np.uint32), k
        if v == 0:
            continue
        # distance of the exact level from the nearest fp32 rounding boundary, in fp32 ulps:
        # far from 1/2 means the fp64 -> fp32 path cannot double-round.
        ulp = mpmath.mpf(float(np.spacing(np.float32(abs(float(v))))))
        frac = abs(v - mpmath.mpf(float(f32))) / ulp
        assert frac < mpmath.mpf("0.49"), (k, frac)


def test_bits_match_scipy_ndtri():
    top = ndtri(_DELTA)
    pos = [ndtri(0.5 + j * (_DELTA - 0.5) / 8) / top for j in range(1, 9)]
    neg = [-ndtri(0.5 + j * (_DELTA - 0.5) / 7) / top for j in range(1, 8)]
    cb2 = np.array(sorted(neg + [0.0] + pos)).astype(np.float32)
    assert np.array_equal(cb2.view(np.uint32), oracle.nf4_codebook().view(np.uint32))


def test_equal_probability_bins():
    """Each half of the type splits its probability range into equal steps (checked with the
    forward normal CDF, not the inverse used to build the table)."""
    cb = oracle.nf4_codebook_f64()
    top = ndtri(_DELTA)
    p = ndtr(cb * top)
    pos_steps = np.diff(p[7:])
    neg_steps = np.diff(p[:8])
    assert np.allclose(pos_steps, pos_steps[0], rtol=1e-9, atol=0)
    assert np.allclose(neg_steps, neg_steps[0], rtol=1e-9, atol=0)
    assert p[15] == pytest.approx(_DELTA, abs=1e-12)
    assert p[0] == pytest.approx(1 - _DELTA, abs=1e-12)
    assert p[7] == 0.5
    # 8 positive steps and 7 negative steps share the same range
    assert pos_steps[0] * 8 == pytest.approx(neg_steps[0] * 7, rel=1e-9)


def test_midpoints_exact_and_the_four_fp32_ties():
    mids = oracle.nf4_midpoints()
    cb = oracle.nf4_codebook().astype(np.float64)
    fmid = (cb[:-1] + cb[1:]) / 2
    for j, m in enumerate(mids):
        assert float(m) == fmid[j]  # fp64 holds every midpoint exactly
    f32_exact = [j for j, m in enumerate(mids) if float(np.float32(float(m))) == m]
    assert f32_exact == [2, 6, 7, 14]
