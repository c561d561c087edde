"""Oracle pins: PDR outlier count and decision, and the BF16-route GEMM.

The pages (gist.science summaries, section 2.C "Purified Delta Refresh")
say only that a block input with a high outlier ratio is computed in full
precision for that step.  The outlier test (|x| above kappa times the token
row's RMS, as x^2 K > kappa^2 sum x^2) and the strict ratio > rho are this
build's reading; the pins check that reading against closed forms and exact
rational arithmetic, not against a retyped formula.
"""
from fractions import Fraction

import numpy as np

from workloads import to_bf16_bits


def _bits(a):
    return to_bf16_bits(np.asarray(a, np.float32))


def test_single_spike_row_boundary(orc):
    # one nonzero element a in a row of K = 64: S = a^2, so it is an outlier
    # iff 64 a^2 > kappa^2 a^2, i.e. kappa < 8 (strict: kappa = 8 is not)
    K = 64
    for a in (1.0, -3.5, 2.0 ** -60, 1.5e30):
        x = np.zeros((1, K), np.float32)
        x[0, 17] = a
        b = _bits(x)
        assert orc.outlier_count(b, 7.9) == 1
        assert orc.outlier_count(b, 7.95) == 1
        assert orc.outlier_count(b, 8.0) == 0
        assert orc.outlier_count(b, 9.0) == 0


def test_constant_magnitude_rows(orc):
    # |x| = c everywhere: x^2 K = K c^2 = S, an outlier iff kappa < 1
    rng = np.random.default_rng(1)
    x = np.where(rng.random((5, 48)) < 0.5, -0.75, 0.75).astype(np.float32)
    b = _bits(x)
    assert orc.outlier_count(b, 0.5) == x.size
    assert orc.outlier_count(b, 0.999) == x.size
    assert orc.outlier_count(b, 1.0) == 0


def test_count_matches_exact_rational(orc):
    # small integers are exact in bf16; the test is decided in exact arithmetic
    rng = np.random.default_rng(2)
    for kappa in (1.5, 2.0, 2.5, 3.0):
        x = rng.integers(-8, 9, (7, 32)).astype(np.float32)
        x[3] = 0
        x[4, :4] = 40
        want = 0
        for row in x:
            S = sum(Fraction(int(v)) ** 2 for v in row)
            for v in row:
                if Fraction(int(v)) ** 2 * len(row) > Fraction(kappa) ** 2 * S:
                    want += 1
        assert orc.outlier_count(_bits(x), kappa) == want, kappa


def test_count_scale_invariant_and_band(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 64)).astype(np.float32)
    x[:, 5] *= 30
    b = _bits(x)
    c = orc.outlier_count(b, 3.0)
    assert 20 <= c < x.size
    for j in (-40, -3, 7, 50):  # power-of-two scaling is exact in bf16
        assert orc.outlier_count(_bits(_bits_f(b) * np.float32(2.0 ** j)), 3.0) == c
    lo, hi = orc.outlier_count_band(b, 3.0, 1e-12)
    assert lo <= c <= hi and hi - lo <= 1


def _bits_f(b):
    from workloads import bf16_bits_to_f32
    return bf16_bits_to_f32(b)


def test_pdr_force_threshold(orc):
    assert orc.pdr_force(11, 100, 0.1)
    assert not orc.pdr_force(10, 100, 0.1)   # equal ratio: not above rho
    assert not orc.pdr_force(0, 100, 0.0)
    assert orc.pdr_force(1, 100, 0.0)
    assert not orc.pdr_force(0, 0, 0.0)      # empty input never forces


def test_gemm_bf16_exact_small_integers(orc):
    rng = np.random.default_rng(4)
    M, N, K = 9, 7, 80
    x = rng.integers(-16, 17, (M, K))
    w = rng.integers(-16, 17, (N, K))
    y, bound = orc.gemm_bf16(_bits(x.astype(np.float32)), _bits(w.astype(np.float32)))
    assert np.array_equal(y, (x @ w.T).astype(np.float64))
    assert np.array_equal(bound, (np.abs(x) @ np.abs(w).T).astype(np.float64))


def test_gemm_bf16_rows_and_rational(orc):
    rng = np.random.default_rng(5)
    M, N, K = 6, 5, 48
    xb = _bits(rng.standard_normal((M, K)).astype(np.float32))
    wb = _bits(rng.standard_normal((N, K)).astype(np.float32) * np.float32(1e-3))
    xf, wf = _bits_f(xb), _bits_f(wb)
    y, b = orc.gemm_bf16(xb, wb)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(float(xf[m, k])) * Fraction(float(wf[n, k])) for k in range(K))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(K) * Fraction(2) ** -52 * Fraction(b[m, n])
    yr, _ = orc.gemm_bf16(xb, wb, rows=np.array([4, 1]))
    assert np.array_equal(yr, y[[4, 1]])
