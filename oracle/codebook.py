"""NF4 codebook: the 16 levels of the 4-bit storage type.

Test infrastructure only (see the package docstring).

Source: "qlora" encyclopedia entry (tonho.wtf), section "como funciona".  The
type is built from quantiles of the standard normal; the tensor is mapped to
[-1, 1] by its absolute maximum, so the levels are normal quantiles divided by
the largest one; each bin holds the same expected number of values (equal
probability steps); the type is asymmetric so that zero is represented
exactly.

The page leaves three choices open.  Readings taken here:

1. The positive side gets 8 levels and the negative side 7 (plus the exact 0),
   16 codes in total.
2. The outermost quantile cannot be the probability-1 point (it is infinite),
   so the probability range stops at delta = 1 - (1/32 + 1/30)/2, the mean of
   the half-bin offsets of a 16-level and a 15-level equal-probability grid.
3. Levels are equally spaced in probability within each half:
     positive  p_j = Phi^-1(1/2 + j (delta - 1/2) / 8),  j = 1..8
     negative  n_j = -Phi^-1(1/2 + j (delta - 1/2) / 7), j = 1..7
   and every level is divided by Phi^-1(delta), so that p_8 = 1 and n_7 = -1.

The fp32 codebook is the round-to-nearest-even of the (high precision) real
values.

Pins (tests/test_oracle_codebook.py): CB[0] = -1, CB[7] = 0, CB[15] = +1,
strictly increasing, 7 negative / 8 positive; the fp32 bits are identical
when Phi^-1 is evaluated by mpmath at 60 digits (rounded exactly from the
high-precision value) and by scipy's ndtri; equal-probability property of the
unnormalised levels.
"""

from fractions import Fraction
from statistics import NormalDist

import numpy as np

_DELTA = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)


def _inv_phi(p: float) -> float:
    # Standard-normal quantile function (stdlib, Wichura's AS241 algorithm).
    return NormalDist().inv_cdf(p)


def nf4_codebook_f64() -> np.ndarray:
    """The 16 NF4 levels in fp64, ascending, before rounding to fp32."""
    top = _inv_phi(_DELTA)
    pos = [_inv_phi(0.5 + j * (_DELTA - 0.5) / 8.0) / top for j in range(1, 9)]
    neg = [-_inv_phi(0.5 + j * (_DELTA - 0.5) / 7.0) / top for j in range(1, 8)]
    levels = sorted(neg + [0.0] + pos)
    return np.array(levels, dtype=np.float64)


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 levels as fp32 (round to nearest even), code k -> CB[k]."""
    return nf4_codebook_f64().astype(np.float32)


def nf4_midpoints() -> list:
    """Exact midpoints (CB[j] + CB[j+1]) / 2 of the fp32 codebook, as Fractions.

    A value x with x / c strictly between midpoints j-1 and j is nearest to
    code j.  Each midpoint of two fp32 numbers needs at most 26 significant
    bits, so it is also exact in fp64.
    """
    cb = nf4_codebook()
    return [(Fraction(float(cb[j])) + Fraction(float(cb[j + 1]))) / 2 for j in range(15)]
