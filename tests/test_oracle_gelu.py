"""Oracle pins: the GELU of the fused producer epilogue (exact erf form).

GELU(x) = x * Phi(x) with Phi the standard normal CDF, so
GELU(x) - GELU(-x) = x (Phi(x) + Phi(-x) = 1), GELU(0) = 0, GELU(x) -> x and
GELU(-x) -> 0 for large x, and GELU(x) / x equals the tabulated Phi(x).
"""
import numpy as np

# standard normal CDF, textbook values
PHI = {-2.0: 0.022750131948179195, -1.0: 0.15865525393145707, 0.5: 0.6914624612740131,
       1.0: 0.8413447460685429, 1.5: 0.9331927987311419, 2.0: 0.9772498680518208,
       3.0: 0.9986501019683699}


def test_gelu_identities(orc):
    xs = np.array([-7.0, -2.5, -1.0, -0.3, 0.3, 1.0, 2.5, 7.0, 31.0])
    g = orc.gelu(xs)
    assert orc.gelu(0.0) == 0.0
    assert np.allclose(g - orc.gelu(-xs), xs, rtol=0, atol=1e-15 * (1 + np.abs(xs)))
    assert orc.gelu(31.0) == 31.0 and abs(orc.gelu(-31.0)) < 1e-200


def test_gelu_tabulated_phi(orc):
    for x, phi in PHI.items():
        assert abs(orc.gelu(x) / x - phi) <= 2e-16, x
    # far negative: x * Phi(x) stays accurate (no cancellation)
    assert abs(orc.gelu(-6.0) / -6.0 - 9.865876450376946e-10) <= 1e-23
