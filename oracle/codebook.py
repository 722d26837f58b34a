"""The 16 NF4 levels of the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

deep-fold README ("Метод" section) stores 4-bit NF4 codes and credits NF4 to
QLoRA; the formula that should follow its colon is lost from the page and no
table of levels is printed.  The levels are therefore built here from the
QLoRA construction (a normal-float data type: quantiles of N(0,1) at evenly
spaced probabilities, with one exact zero, scaled to [-1, 1]):

* positive side: 8 levels Phi^-1(p) at p = delta + (1/2 - delta) * i / 8,
  i = 0..7 (nine evenly spaced probabilities from delta to 1/2; the last one
  maps to 0 and is dropped);
* negative side: 7 levels -Phi^-1(p) at p = delta + (1/2 - delta) * i / 7,
  i = 0..6;
* one exact zero;
* all divided by Phi^-1(delta), so the extremes are exactly -1 and +1.

delta, the outermost probability, is read as 1 - (1/32 + 1/30) / 2: half a
bin in from the tail, averaged between the 16-bin (positive) and 15-bin
(negative) partitions.  The levels are computed in float64 and rounded once
to binary32 (round to nearest even); those 16 binary32 values ARE the
codebook.  Level values: parity unpinned by the pages (no table printed);
their construction is pinned in tests by an independent inverse-CDF.
"""

import numpy as np
from scipy.special import ndtri

NF4_DELTA = 1.0 - (1.0 / 32.0 + 1.0 / 30.0) / 2.0


def nf4_levels_f64():
    """The 16 levels in float64, ascending, before the binary32 rounding."""
    d = NF4_DELTA
    pos = ndtri(d + (0.5 - d) * np.arange(8, dtype=np.float64) / 8.0)
    neg = -ndtri(d + (0.5 - d) * np.arange(7, dtype=np.float64) / 7.0)
    top = ndtri(d)
    lv = np.concatenate([neg / top, [0.0], pos / top])
    return np.sort(lv)


def nf4_levels_f32():
    """The codebook: 16 binary32 levels, ascending; c[0] = -1, c[7] = +0, c[15] = +1."""
    return nf4_levels_f64().astype(np.float32)
