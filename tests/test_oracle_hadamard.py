"""Pins for the oracle's 16-point block Hadamard (Sylvester order, scaled 1/4).

Pinned against: the Sylvester matrix written from its closed form
(-1)^popcount(i & j), orthonormality H H^T = I (exact), equality with the
dense product for small-integer inputs, the involution property, Parseval,
and block placement along K inside the quantizers.
"""
import numpy as np

import workloads


def _sylvester16():
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def _matrix(orc):
    cols = [orc.fwht16(np.eye(16, dtype=np.float32)[j]) for j in range(16)]
    return np.stack(cols, axis=1).astype(np.float64)


def test_fwht_is_sylvester_over_four(orc):
    H = _matrix(orc)
    assert np.array_equal(H, _sylvester16() / 4)


def test_fwht_orthonormal_exact(orc):
    H = _matrix(orc)
    assert np.array_equal(H @ H.T, np.eye(16))


def test_fwht_dense_and_involution_small_ints(orc):
    rng = np.random.default_rng(1)
    S = _sylvester16()
    for _ in range(200):
        x = rng.integers(-40, 41, 16).astype(np.float32)
        y = orc.fwht16(x)
        assert np.array_equal(y.astype(np.float64), S @ x.astype(np.float64) / 4)
        assert np.array_equal(orc.fwht16(y), x)


def test_fwht_parseval(orc):
    rng = np.random.default_rng(2)
    for _ in range(200):
        x = rng.standard_normal(16).astype(np.float32) * np.float32(rng.uniform(1e-3, 1e3))
        y = orc.fwht16(x)
        nx = np.linalg.norm(x.astype(np.float64))
        ny = np.linalg.norm(y.astype(np.float64))
        assert abs(nx - ny) <= 4e-7 * nx


def test_rotation_acts_per_16_block_along_k(orc):
    # one nonzero at column 16*j + i spreads over block j only, with the signs
    # of Sylvester column i; every other block stays zero
    S = _sylvester16()
    K = 64
    for j in range(K // 16):
        for i in (0, 5, 15):
            x = np.zeros((1, K), np.float32)
            x[0, 16 * j + i] = 8.0
            q, s = orc.quant_int8(workloads.to_bf16_bits(x))
            assert s[0] == np.float32(2.0) / np.float32(127.0)
            expect = np.zeros(K, np.int8)
            expect[16 * j:16 * j + 16] = (127 * S[:, i]).astype(np.int8)
            assert np.array_equal(q[0], expect), (j, i)
