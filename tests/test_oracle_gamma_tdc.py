"""Pins for the oracle's Gamma predictor, router and Temporal Delta Cache.

Pinned against: closed forms of the relative L1 distance (Gamma(X, X) = 0,
Gamma(X, 0) = 1, Gamma(X, 2X) = 1, Gamma(X, -X) = 2, power-of-two scale
invariance), exact summation (math.fsum), the router's threshold on both
sides and at the tie, the INT8 fallback, the skip output as an elementwise
bf16 sum, and the refresh period floor(delta/d) + 1 of the accumulated-error
gate.
"""
import math

import numpy as np
import pytest

import workloads
from workloads import bf16_bits_to_f32, to_bf16_bits


def _x(seed, M=33, K=64):
    return workloads.activations(np.random.default_rng(seed), M, K)


def test_gamma_closed_forms(orc):
    x = _x(30)
    xf = bf16_bits_to_f32(x)
    assert orc.gamma(orc.gamma_sums(x, x)) == 0.0
    assert orc.gamma(orc.gamma_sums(x, np.zeros_like(x))) == 1.0
    assert orc.gamma(orc.gamma_sums(x, to_bf16_bits(2 * xf))) == 1.0
    assert orc.gamma(orc.gamma_sums(x, to_bf16_bits(-xf))) == 2.0
    z = np.zeros_like(x)
    assert orc.gamma(orc.gamma_sums(z, z)) == 0.0
    assert orc.gamma(orc.gamma_sums(z, x)) == math.inf


def test_gamma_power_of_two_invariance(orc):
    x, y = _x(31), _x(32)
    g = orc.gamma(orc.gamma_sums(x, y))
    for c in (0.25, 8.0):
        xs = to_bf16_bits(bf16_bits_to_f32(x) * np.float32(c))
        ys = to_bf16_bits(bf16_bits_to_f32(y) * np.float32(c))
        assert orc.gamma(orc.gamma_sums(xs, ys)) == g


def test_gamma_sums_exact_summation(orc):
    x, y = _x(33), _x(34)
    xf, yf = bf16_bits_to_f32(x).ravel(), bf16_bits_to_f32(y).ravel()
    s = orc.gamma_sums(x, y)
    s1 = math.fsum(float(v) for v in np.abs(yf - xf))   # fp32 differences, exact sum
    s2 = math.fsum(float(v) for v in np.abs(xf))
    assert abs(s[0] - s1) <= 1e-12 * s1 and abs(s[1] - s2) <= 1e-12 * s2


def test_route_threshold_both_sides_tie_and_missing(orc):
    alpha = np.array([2.0, 0.5, 1.0])
    beta = np.array([0.1, -0.05, 0.0])
    tau = 0.3
    # Gamma at which each linear's E crosses tau: (tau - beta) / alpha
    for l in range(3):
        gc = (tau - beta[l]) / alpha[l]
        for g, want in ((gc * 1.01, orc.ROUTE_INT8), (gc * 0.99, orc.ROUTE_NVFP4)):
            _, e, r = orc.route(np.array([g, 1.0]), alpha, beta, tau)
            assert r[l] == want
            assert e[l] == alpha[l] * g + beta[l]
    # exact tie (E == tau) goes to NVFP4: alpha=1, beta=0, Gamma = 0.25 = tau
    _, e, r = orc.route(np.array([1.0, 4.0]), np.array([1.0]), np.array([0.0]), 0.25)
    assert e[0] == 0.25 and r[0] == orc.ROUTE_NVFP4
    g, e, r = orc.route(None, alpha, beta, tau)
    assert math.isnan(g) and np.all(r == orc.ROUTE_INT8)


def test_tdc_skip_is_elementwise_bf16_sum(orc):
    x, d = _x(35), _x(36)
    out = orc.tdc_skip(x, d)
    want = to_bf16_bits(bf16_bits_to_f32(x) + bf16_bits_to_f32(d))
    assert np.array_equal(out, want)


def test_tdc_refresh_delta_and_sums(orc):
    x, y, dprev = _x(37), _x(38), _x(39)
    delta = dprev.copy()
    s = orc.tdc_refresh(x, y, delta, True)
    xf, yf = bf16_bits_to_f32(x), bf16_bits_to_f32(y)
    want = to_bf16_bits(yf - xf)
    assert np.array_equal(delta, want)
    assert np.array_equal(s[:2], orc.gamma_sums(x, y))
    dn, dp = bf16_bits_to_f32(want).ravel(), bf16_bits_to_f32(dprev).ravel()
    s3 = math.fsum(float(v) for v in np.abs(dn - dp))
    s4 = math.fsum(float(v) for v in np.abs(dp))
    assert abs(s[2] - s3) <= 1e-12 * s3 and abs(s[3] - s4) <= 1e-12 * s4
    delta2 = dprev.copy()
    s_first = orc.tdc_refresh(x, y, delta2, False)
    assert s_first[2] == 0 and s_first[3] == 0 and np.array_equal(delta2, want)


def _run_schedule(orc, steps, eps, dacc, block, x0, drift):
    """Drive decide/skip/refresh/commit for one block; returns the skip pattern."""
    st = orc.tdc_new()
    delta = np.zeros_like(x0)
    x = x0
    pattern = []
    for t in range(steps):
        if orc.tdc_decide(st, eps, dacc):
            orc.tdc_skip(x, delta)
            orc.tdc_commit_skip(st)
            pattern.append(1)
        else:
            s = orc.tdc_refresh(x, block(x), delta, bool(st.delta_valid))
            orc.tdc_commit_refresh(st, s)
            pattern.append(0)
        x = drift(x, t)
    return pattern, st


def test_tdc_constant_residual_always_skips_after_warmup(orc):
    # out = in + c with c exactly representable: every delta equals c, d = 0
    x0 = to_bf16_bits(np.round(np.random.default_rng(40).standard_normal((8, 32)) * 8) / 8)
    c = np.float32(0.5)
    block = lambda x: to_bf16_bits(bf16_bits_to_f32(x) + c)
    drift = lambda x, t: to_bf16_bits(bf16_bits_to_f32(x) + np.float32(1.0))
    pattern, st = _run_schedule(orc, 12, 1e-3, 1e-3, block, x0, drift)
    assert pattern == [0, 0] + [1] * 10
    assert st.d == 0.0 and st.acc == 0.0


def test_tdc_refresh_period_from_accumulated_error(orc):
    # constant d = 2^-5 and delta_acc = 3 * 2^-5: 3 skips, then a refresh
    st = orc.tdc_new()
    st.n_refresh, st.delta_valid, st.d, st.acc = 2, 1, 2.0 ** -5, 0.0
    pattern = []
    for _ in range(12):
        if orc.tdc_decide(st, 1.0, 3 * 2.0 ** -5):
            orc.tdc_commit_skip(st)
            pattern.append(1)
        else:
            st.acc = 0.0          # a refresh with the same d
            st.n_refresh += 1
            pattern.append(0)
    assert pattern == [1, 1, 1, 0] * 3
    # general closed form floor(delta/d) + 1
    for d, dacc in ((0.1, 0.35), (0.25, 1.0), (0.3, 0.2)):
        st = orc.tdc_new()
        st.n_refresh, st.delta_valid, st.d = 2, 1, d
        skips = 0
        while orc.tdc_decide(st, 1.0, dacc):
            orc.tdc_commit_skip(st)
            skips += 1
        assert skips == math.floor(dacc / d + 1e-12)


@pytest.mark.parametrize("eps,dacc,want", [(0.0, math.inf, "never"),
                                           (math.inf, math.inf, "always")])
def test_tdc_gate_extremes(orc, eps, dacc, want):
    rng = np.random.default_rng(41)
    x0 = workloads.activations(rng, 8, 32)
    block = lambda x: to_bf16_bits(bf16_bits_to_f32(x) * np.float32(1.5))
    drift = lambda x, t: to_bf16_bits(bf16_bits_to_f32(x) + np.float32(0.02) *
                                      rng.standard_normal(x.shape).astype(np.float32))
    pattern, _ = _run_schedule(orc, 10, eps, dacc, block, x0, drift)
    if want == "never":
        assert pattern == [0] * 10
    else:
        assert pattern == [0, 0] + [1] * 8


def test_tdc_commit_sets_d_gamma(orc):
    st = orc.tdc_new()
    orc.tdc_commit_refresh(st, np.array([1.0, 4.0, 0.0, 0.0]))
    assert st.d == math.inf and st.gamma == 0.25 and st.gamma_valid == 1
    orc.tdc_commit_refresh(st, np.array([3.0, 4.0, 1.0, 8.0]))
    assert st.d == 0.125 and st.n_refresh == 2 and st.acc == 0.0
    orc.tdc_commit_skip(st)
    assert st.acc == 0.125 and st.gamma_valid == 0
