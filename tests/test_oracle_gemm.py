"""Pins for the oracle's INT8 and NVFP4 GEMMs.

Pinned against: brute force in exact Python integers / rationals on tiny
shapes, the scaled-identity special case, zero tensor scales, row sampling
consistency and the int32 range at the largest K.
"""
from fractions import Fraction

import numpy as np
import pytest


def _rand_int8(rng, shape):
    return rng.integers(-127, 128, shape).astype(np.int8)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (5, 7, 32), (33, 17, 48), (64, 40, 64)])
def test_int8_bruteforce(orc, M, N, K):
    rng = np.random.default_rng(M * 1000 + N)
    qa, qw = _rand_int8(rng, (M, K)), _rand_int8(rng, (N, K))
    sa = rng.uniform(1e-3, 1, M).astype(np.float32)
    sw = rng.uniform(1e-3, 1, N).astype(np.float32)
    acc, y = orc.gemm_int8(qa, sa, qw, sw)
    for m in range(M):
        for n in range(N):
            exact = sum(int(a) * int(b) for a, b in zip(qa[m], qw[n]))
            assert acc[m, n] == exact
            want = (np.float32(exact) * sa[m]) * sw[n]
            assert y[m, n] == want


def test_int8_scaled_identity(orc):
    rng = np.random.default_rng(20)
    K = 64
    qa = _rand_int8(rng, (10, K))
    qw = (127 * np.eye(K)).astype(np.int8)
    acc, y = orc.gemm_int8(qa, np.ones(10, np.float32), qw, np.ones(K, np.float32))
    assert np.array_equal(acc, 127 * qa.astype(np.int32))


def test_int8_rows_subset_and_range(orc):
    rng = np.random.default_rng(21)
    M, N, K = 30, 9, 12288
    qa = np.full((M, K), 127, np.int8)
    qa[1::2] = -127
    qw = np.full((N, K), 127, np.int8)
    sa = np.ones(M, np.float32)
    sw = np.ones(N, np.float32)
    acc, y = orc.gemm_int8(qa, sa, qw, sw)
    assert acc[0, 0] == 127 * 127 * K and acc[1, 0] == -127 * 127 * K
    rows = np.array([29, 0, 7])
    acc2, y2 = orc.gemm_int8(qa, sa, qw, sw, rows=rows)
    assert np.array_equal(acc2, acc[rows]) and np.array_equal(y2, y[rows])


def _exact_nvfp4(orc, ca, sa, ga, cw, sw, gw):
    va = orc.nibbles(ca)
    vw = orc.nibbles(cw)
    M, K = va.shape
    N = vw.shape[0]
    E2 = [Fraction(orc.e2m1_value(c)) for c in range(16)]
    E4 = [Fraction(orc.e4m3_value(c)) for c in range(0x7F)]
    y = np.empty((M, N))
    b = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            tab = Fraction(0)
            for k in range(K):
                a = E2[va[m, k]] * E4[sa[m, k // 16]]
                w = E2[vw[n, k]] * E4[sw[n, k // 16]]
                tot += a * w
                tab += abs(a * w)
            y[m, n] = float(tot * Fraction(float(ga)) * Fraction(float(gw)))
            b[m, n] = float(tab * Fraction(float(ga)) * Fraction(float(gw)))
    return y, b


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (3, 4, 32), (6, 5, 64)])
def test_nvfp4_bruteforce_rational(orc, M, N, K):
    rng = np.random.default_rng(K + M)
    ca = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    cw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = rng.integers(0, 0x7F, (M, K // 16)).astype(np.uint8)
    sw = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    ga, gw = 0.0123, 3.5e-3
    y, b = orc.gemm_nvfp4(ca, sa, ga, cw, sw, gw)
    ye, be = _exact_nvfp4(orc, ca, sa, np.float32(ga), cw, sw, np.float32(gw))
    assert np.allclose(y, ye, rtol=1e-14, atol=1e-14 * be.max())
    assert np.allclose(b, be, rtol=1e-14, atol=0)
    assert np.all(np.abs(y) <= b * (1 + 1e-14))


def test_nvfp4_identity_weight(orc):
    # W row n holds +1 at k = n (code 2) with block scale 1.0 (E4M3 0x38), gw = 1:
    # y[m, n] = value(a[m, n]) * scale_a * ga
    rng = np.random.default_rng(22)
    M, K = 7, 32
    ca = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    sa = rng.integers(1, 0x7F, (M, K // 16)).astype(np.uint8)
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 2
    cw = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sw = np.full((K, K // 16), 0x38, np.uint8)
    y, _ = orc.gemm_nvfp4(ca, sa, 0.5, cw, sw, 1.0)
    va = np.vectorize(orc.e2m1_value)(orc.nibbles(ca))
    sc = np.repeat(np.vectorize(orc.e4m3_value)(sa), 16, axis=1)
    assert np.array_equal(y, va * sc * 0.5)


def test_nvfp4_zero_tensor_scale_and_rows(orc):
    rng = np.random.default_rng(23)
    M, N, K = 9, 6, 48
    ca = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    cw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = rng.integers(0, 0x7F, (M, K // 16)).astype(np.uint8)
    sw = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    y0, b0 = orc.gemm_nvfp4(ca, sa, 0.0, cw, sw, 1.0)
    assert not y0.any() and not b0.any()
    y, b = orc.gemm_nvfp4(ca, sa, 0.25, cw, sw, 2.0)
    rows = np.array([8, 3])
    y2, b2 = orc.gemm_nvfp4(ca, sa, 0.25, cw, sw, 2.0, rows=rows)
    assert np.array_equal(y2, y[rows]) and np.array_equal(b2, b[rows])
