"""Host-side pins of the router fit (no GPU): least squares recovers an exact
linear model, a shared Gamma column broadcasts over linears, and degenerate
input is rejected."""
import numpy as np
import pytest

from dynamic_mixed_precision_amd.calibrate import fit_router


def test_fit_recovers_exact_line():
    g = np.array([0.05, 0.1, 0.2, 0.4, 0.8])
    a, b, rms = fit_router(g, 0.3 * g + 0.02)
    assert abs(a[0] - 0.3) < 1e-12 and abs(b[0] - 0.02) < 1e-12 and rms[0] < 1e-14


def test_fit_per_linear_with_shared_gamma():
    rng = np.random.default_rng(0)
    g = rng.random(40)
    alpha = np.array([0.5, -0.1, 2.0])
    beta = np.array([0.01, 0.3, -0.2])
    e = g[:, None] * alpha + beta
    a, b, rms = fit_router(g, e)
    assert np.allclose(a, alpha, atol=1e-12) and np.allclose(b, beta, atol=1e-12)
    assert np.all(rms < 1e-13)


def test_fit_noise_is_least_squares():
    # residual orthogonal to both regressors (the normal equations)
    rng = np.random.default_rng(1)
    g = rng.random(200)
    e = 0.2 * g + 0.05 + 0.01 * rng.standard_normal(200)
    a, b, _ = fit_router(g, e)
    r = e - (a[0] * g + b[0])
    assert abs(r.sum()) < 1e-10 and abs((r * g).sum()) < 1e-10


def test_fit_rejects_bad_input():
    with pytest.raises(ValueError):
        fit_router([0.1], [0.2])
    with pytest.raises(ValueError):
        fit_router(np.zeros((3, 2)), np.zeros((3, 3)))
