"""Element-wise check of bf16 weights after a step, shared by the GPU tests.

A plain "≤ 1 ulp of the oracle's rounding" rule is wrong where W0 − lr·sc·O
cancels towards zero (there the bf16 ulp is far below the update's own
error), so updated weights are checked in two parts:
  * every weight is the round-to-nearest-even of W0 − lrsc·Õ for some Õ
    within ±band·rms(O) of the oracle's update O;
  * the fraction of weights that differ from round(W0 − lrsc·O) stays below
    the fraction an update error at the 2e-2 relative bound would produce.
"""
import numpy as np

import oracle

TOL_BF16 = 2e-2


def weights_consistent(W0, got, O, lrsc, band=0.1, decay=1.0, tol=TOL_BF16):
    """Returns (every weight inside the band, fraction differing from the
    oracle's rounding, the fraction an update error of relative size `tol`
    would produce)."""
    rms = float(np.sqrt(np.mean(O * O)))
    b = band * rms
    lo = oracle.bf16_round(decay * W0 - lrsc * (O + b))
    hi = oracle.bf16_round(decay * W0 - lrsc * (O - b))
    ok = bool(np.all((got >= lo) & (got <= hi)))
    frac = float(np.mean(got != oracle.bf16_round(decay * W0 - lrsc * O)))
    # an error of per-element rms tol·rms(O) moves an element across a bf16
    # rounding boundary with probability ≈ 2·lrsc·tol·rms / ulp (capped at 1)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(got), 2.0 ** -126))) - 7)
    expect = float(np.mean(np.minimum(1.0, 2.0 * lrsc * tol * rms / ulp)))
    return ok, frac, expect
