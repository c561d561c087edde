"""Pins for the oracle's INT8 / NVFP4 activation quantizers and weight prep.

Pinned against: exact round trips of tensors built on the quantization grid
(scale a power of two for INT8; g = 1 and every block amax = 6 * scale for
NVFP4), NVFP4 scales and codes at g != 1 against exact rational RNE, zero
and spike special cases, RNE error bounds, row-permutation
equivariance, the Hadamard composed from its closed form, and X W^T
invariance of the rotation.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from workloads import bf16_bits_to_f32, to_bf16_bits


def _sylvester16():
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def _rotate_exact(x):
    """Block Hadamard via the dense closed form (exact for small integers)."""
    M, K = x.shape
    H = _sylvester16() / 4
    return (x.reshape(M, K // 16, 16) @ H.T).reshape(M, K)


# ---- INT8 -----------------------------------------------------------------

def test_int8_roundtrip_on_grid(orc):
    rng = np.random.default_rng(3)
    M, K = 37, 96
    q = rng.integers(-127, 128, (M, K)).astype(np.int8)
    q[np.arange(M), rng.integers(0, K, M)] = rng.choice([-127, 127], M)
    s = np.ldexp(1.0, -rng.integers(0, 12, M)).astype(np.float32)
    x = to_bf16_bits(q.astype(np.float32) * s[:, None])
    q2, s2 = orc.quant_int8(x, flags=orc.NO_HADAMARD)
    # s = amax/127 with amax = 127 * 2^-k: exact
    assert np.array_equal(s2, s)
    assert np.array_equal(q2, q)


def test_int8_zero_row_and_spike(orc):
    K = 48
    x = np.zeros((3, K), np.float32)
    x[1, 7] = -3.5
    x[2, :] = 0.25
    q, s = orc.quant_int8(to_bf16_bits(x), flags=orc.NO_HADAMARD)
    assert s[0] == 0 and not q[0].any()
    assert q[1, 7] == -127 and np.count_nonzero(q[1]) == 1
    assert s[1] == np.float32(3.5) / np.float32(127)
    assert np.all(q[2] == 127)


def test_int8_rne_error_bound(orc):
    rng = np.random.default_rng(4)
    x = workloads.activations(rng, 64, 256)
    q, s = orc.quant_int8(x)
    xt = np.stack([np.concatenate([orc.fwht16(r[j:j + 16]) for j in range(0, 256, 16)])
                   for r in bf16_bits_to_f32(x)]).astype(np.float64)
    amax = np.abs(xt).max(axis=1)
    assert np.allclose(s, amax / 127, rtol=2e-7, atol=0)
    err = np.abs(q.astype(np.float64) * s[:, None] - xt)
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-5) + 1e-6 * amax[:, None])
    assert np.all(np.abs(q).max(axis=1) == 127)


def test_int8_rows_permute(orc):
    rng = np.random.default_rng(5)
    x = workloads.activations(rng, 50, 128)
    perm = rng.permutation(50)
    q, s = orc.quant_int8(x)
    qp, sp = orc.quant_int8(np.ascontiguousarray(x[perm]))
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])


def test_int8_hadamard_is_block_rotation(orc):
    rng = np.random.default_rng(6)
    x = rng.integers(-7, 8, (20, 64)).astype(np.float32)
    xt = _rotate_exact(x.astype(np.float64)).astype(np.float32)
    a = orc.quant_int8(to_bf16_bits(x))
    b = orc.quant_int8(to_bf16_bits(xt), flags=orc.NO_HADAMARD)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---- NVFP4 ----------------------------------------------------------------

def _nvfp4_grid_tensor(orc, rng, M, K):
    """Tensor with g = 1: values val(c) * dec(e_b), every block holding a +-6."""
    nb = K // 16
    codes = rng.integers(0, 16, (M, K)).astype(np.uint8)
    pos = rng.integers(0, 16, (M, nb))
    for m in range(M):
        for b in range(nb):
            codes[m, 16 * b + pos[m, b]] = rng.choice([7, 15])
    e = rng.integers(1, 0x7F, (M, nb)).astype(np.uint8)
    e[0, 0] = 0x7E  # tensor amax = 6 * 448 = 2688 -> g = 1
    val = np.vectorize(orc.e2m1_value)(codes).astype(np.float64)
    dec = np.vectorize(orc.e4m3_value)(e).astype(np.float64)
    x = val * np.repeat(dec, 16, axis=1)
    xb = to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(xb).astype(np.float64), x)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return xb, packed, e


def test_nvfp4_roundtrip_on_grid(orc):
    rng = np.random.default_rng(7)
    xb, codes, e = _nvfp4_grid_tensor(orc, rng, 9, 80)
    c2, s2, g = orc.quant_nvfp4(xb, flags=orc.NO_HADAMARD)
    assert g == 1.0
    assert np.array_equal(s2, e)
    assert np.array_equal(c2, codes)


def test_nvfp4_all_zero(orc):
    c, s, g = orc.quant_nvfp4(np.zeros((4, 32), np.uint16))
    assert g == 0.0 and not c.any() and not s.any()


def test_nvfp4_properties_random(orc):
    rng = np.random.default_rng(8)
    M, K = 48, 256
    x = workloads.activations(rng, M, K)
    c, s, g = orc.quant_nvfp4(x)
    xt = np.stack([np.concatenate([orc.fwht16(r[j:j + 16]) for j in range(0, K, 16)])
                   for r in bf16_bits_to_f32(x)]).astype(np.float64)
    A = np.abs(xt).max()
    assert g == np.float32(np.float32(A) / np.float32(2688.0))
    assert np.all(s <= 0x7E)                       # non-negative, finite, <= 448
    codes = orc.nibbles(c)
    val = np.vectorize(orc.e2m1_value)(codes).astype(np.float64)
    S = np.vectorize(orc.e4m3_value)(s).astype(np.float64) * g
    S16 = np.repeat(S, 16, axis=1)
    # block amax maps to the top code (scale ~ amax/6 up to E4M3 rounding)
    blk_max = np.abs(val).reshape(M, K // 16, 16).max(axis=2)
    normal = S >= 2.0 ** -6 * g
    assert np.all(blk_max[normal] == 6.0)
    # dequantization error: at most half the largest E2M1 gap (1.0) times S,
    # plus whatever saturation clipped
    err = np.abs(val * S16 - xt)
    clip = np.maximum(np.abs(xt) - 6 * S16, 0)
    assert np.all(err <= 1.0 * S16 * (1 + 1e-6) + clip)


def _rne_on_grid(q, grid):
    """Index of the nearest value of the ascending exact grid to q >= 0 (ties to
    the even index, values above the top saturate), and whether q lies within
    a relative 2^-20 of a midpoint (where fp32 evaluation may round either way)."""
    if q >= grid[-1]:
        return len(grid) - 1, False
    hi = next(i for i, v in enumerate(grid) if v >= q)
    if grid[hi] == q or hi == 0:
        return hi, False
    lo = hi - 1
    mid = (grid[lo] + grid[hi]) / 2
    near = abs(q - mid) <= q * Fraction(1, 2 ** 20)
    if q == mid:
        return (lo if lo % 2 == 0 else hi), near
    return (lo if q < mid else hi), near


def _e4m3_grid():
    vals = []
    for c in range(0x7F):  # non-negative finite codes, ascending
        e, m = c >> 3, c & 7
        vals.append(Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


def test_nvfp4_scales_and_codes_against_exact_rationals(orc):
    """At g != 1, on blocks spanning the E4M3 range: every block scale is the
    E4M3 RNE of the exact rational 448 * a_b / A and every code the E2M1 RNE
    of x / (E4M3(...) * A / 2688), except within fp32 rounding distance of a
    midpoint (the pages fix no evaluation order; those cases are counted)."""
    rng = np.random.default_rng(31)
    M, K = 24, 384
    x = workloads.activations(rng, M, K)
    c, s, g = orc.quant_nvfp4(x, flags=orc.NO_HADAMARD)
    xf = bf16_bits_to_f32(x)
    A = Fraction(float(np.abs(xf).max()))
    assert g == np.float32(np.float32(float(A)) / np.float32(2688.0)) and g != 1.0
    e4 = _e4m3_grid()
    e2 = [Fraction(v, 2) for v in (0, 1, 2, 3, 4, 6, 8, 12)]
    codes = orc.nibbles(c)
    skipped = checked = 0
    for m in range(M):
        for b in range(K // 16):
            blk = xf[m, 16 * b:16 * b + 16]
            ab = Fraction(float(np.abs(blk).max()))
            want, near = _rne_on_grid(448 * ab / A, e4)
            if near:
                skipped += 1
                continue
            assert s[m, b] == want, (m, b)
            S = e4[want] * A / 2688
            if float(S) < np.finfo(np.float32).tiny:
                assert not codes[m, 16 * b:16 * b + 16].any()
                continue
            for i in range(16):
                v = Fraction(float(blk[i]))
                k, near = _rne_on_grid(abs(v) / S, e2)
                if near:
                    skipped += 1
                    continue
                sign = 8 if np.signbit(blk[i]) else 0
                assert codes[m, 16 * b + i] == (k | sign), (m, b, i)
                checked += 1
    assert len(set(s.ravel().tolist())) > 20          # many scale codes exercised
    assert checked > 0.95 * M * K and skipped < 0.01 * M * K


def test_nvfp4_hadamard_is_block_rotation(orc):
    rng = np.random.default_rng(9)
    x = rng.integers(-7, 8, (12, 64)).astype(np.float32)
    xt = _rotate_exact(x.astype(np.float64)).astype(np.float32)
    a = orc.quant_nvfp4(to_bf16_bits(x))
    b = orc.quant_nvfp4(to_bf16_bits(xt), flags=orc.NO_HADAMARD)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


def test_quant_rejects_bad_k(orc):
    with pytest.raises(ValueError):
        orc.quant_int8(np.zeros((2, 24), np.uint16))
    with pytest.raises(ValueError):
        orc.quant_nvfp4(np.zeros((2, 40), np.uint16))


# ---- weight preparation ---------------------------------------------------

def test_prep_weight_nvfp4_part_is_quantizer(orc):
    rng = np.random.default_rng(10)
    w = workloads.weight(rng, 40, 64)
    p = orc.prep_weight(w)
    c, s, g = orc.quant_nvfp4(w)
    assert np.array_equal(p["cw"], c) and np.array_equal(p["sw"], s) and p["gw"] == g


def test_prep_weight_int8_from_nvfp4(orc):
    rng = np.random.default_rng(11)
    N, K = 40, 64
    p = orc.prep_weight(workloads.weight(rng, N, K))
    val = np.vectorize(orc.e2m1_value)(orc.nibbles(p["cw"])).astype(np.float32)
    dec = np.repeat(np.vectorize(orc.e4m3_value)(p["sw"]).astype(np.float32), 16, axis=1)
    wd = (val * dec) * np.float32(p["gw"])
    amax = np.abs(wd).max(axis=1).astype(np.float64)
    assert np.allclose(p["sw_row"], amax / 127, rtol=2e-7, atol=0)
    err = np.abs(p["qw"] * p["sw_row"][:, None].astype(np.float64) - wd)
    assert np.all(err <= 0.5 * p["sw_row"][:, None] * (1 + 1e-5) + 1e-6 * amax[:, None])
    # the requantized weight keeps the NVFP4 weight's zero pattern and signs
    assert np.array_equal(np.sign(p["qw"]), np.sign(np.round(wd / p["sw_row"][:, None])))


def _pack_nibbles(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_w8_from_nvfp4_closed_form(orc):
    # g = 127/128 and a row amax of 4 * g = 127/32 make 127/amax exactly 32 in
    # fp32, so every code is the round-half-even of v * s * 127/4 in exact
    # rational arithmetic (E2M1 values from the OCP table; E4M3 0x38 = 1.0,
    # 0x30 = 0.5).  v*s = 2 lands on the tie 63.5 -> 64.
    from fractions import Fraction
    e2m1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    K = 32
    row0 = [0, 1, 2, 3, 4, 5, 6, 9, 10, 11, 12, 13, 14, 8, 1, 6,    # group 0: scale 1.0
            7, 15, 5, 13, 3, 11, 1, 9, 4, 12, 2, 10, 6, 14, 0, 8]   # group 1: scale 0.5
    row1 = [c ^ 8 for c in row0]                                    # every sign flipped
    row2 = [0] * K                                                  # all zero
    codes = np.array([row0, row1, row2], np.uint8)
    scales = np.array([[0x38, 0x30]] * 3, np.uint8)
    g = Fraction(127, 128)
    qw, swr = orc.w8_from_nvfp4(_pack_nibbles(codes), scales, float(g))
    for n in range(2):
        for k in range(K):
            c = int(codes[n, k])
            v = e2m1[c & 7] * (-1 if c & 8 else 1)
            s = Fraction(1) if k < 16 else Fraction(1, 2)
            want = round(v * s * g * 32)  # Fraction.__round__ ties to even
            assert qw[n, k] == want, (n, k, c, want, qw[n, k])
        assert swr[n] == np.float32(1 / 32)
    assert np.all(qw[2] == 0) and swr[2] == 0.0
    assert qw[0, 4] == 64  # the tie: v*s = 2


def test_w8_from_nvfp4_matches_prep_weight(orc):
    rng = np.random.default_rng(14)
    p = orc.prep_weight(workloads.weight(rng, 33, 96))
    qw, swr = orc.w8_from_nvfp4(p["cw"], p["sw"], p["gw"])
    assert np.array_equal(qw, p["qw"]) and np.array_equal(swr.view(np.uint32), p["sw_row"].view(np.uint32))


def test_prep_weight_direct_is_int8_quant(orc):
    rng = np.random.default_rng(12)
    w = workloads.weight(rng, 24, 48)
    p = orc.prep_weight(w, orc.W8_DIRECT)
    q, s = orc.quant_int8(w)
    assert np.array_equal(p["qw"], q) and np.array_equal(p["sw_row"], s)


def test_rotation_preserves_xwt_exactly(orc):
    # (X H)(W H)^T = X W^T: exact for small integers without quantization
    rng = np.random.default_rng(13)
    x = rng.integers(-6, 7, (8, 64)).astype(np.float64)
    w = rng.integers(-6, 7, (5, 64)).astype(np.float64)
    xr = np.stack([np.concatenate([orc.fwht16(r[j:j + 16]) for j in range(0, 64, 16)]) for r in x])
    wr = np.stack([np.concatenate([orc.fwht16(r[j:j + 16]) for j in range(0, 64, 16)]) for r in w])
    assert np.array_equal(xr.astype(np.float64) @ wr.T.astype(np.float64), x @ w.T)


def test_rotated_quantized_linear_tracks_float(orc):
    rng = np.random.default_rng(14)
    M, N, K = 64, 48, 256
    x = workloads.activations(rng, M, K)
    w = workloads.weight(rng, N, K)
    ref = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    p = orc.prep_weight(w)
    qa, sa = orc.quant_int8(x)
    _, y8 = orc.gemm_int8(qa, sa, p["qw"], p["sw_row"])
    ca, sca, ga = orc.quant_nvfp4(x)
    y4, _ = orc.gemm_nvfp4(ca, sca, ga, p["cw"], p["sw"], p["gw"])
    rel8 = np.linalg.norm(y8 - ref) / np.linalg.norm(ref)
    rel4 = np.linalg.norm(y4 - ref) / np.linalg.norm(ref)
    assert rel8 < 0.12 and rel4 < 0.2
    # INT8 activations over the NVFP4-derived weight beat all-NVFP4
    assert rel8 < rel4


def test_int8_row_without_finite_reciprocal(orc):
    # 127/amax must be a finite fp32: amax at or below 127/FLT_MAX (~3.7e-37)
    # quantizes as a zero row; just above, the row spans +-127 as usual
    K = 32
    x = np.zeros((3, K), np.float32)
    x[0, 3] = 1e-38                      # bf16 subnormal-range value: 127/a overflows
    x[1, 5] = -2e-37                     # 127/a = 6.35e38 > FLT_MAX: overflows
    x[2, 7] = 4e-37                      # 127/a = 3.2e38: finite
    q, s = orc.quant_int8(to_bf16_bits(x), flags=orc.NO_HADAMARD)
    assert s[0] == 0 and not q[0].any()
    assert s[1] == 0 and not q[1].any()
    assert s[2] > 0 and q[2, 7] == 127 and np.count_nonzero(q[2]) == 1


# ---- non-finite inputs ------------------------------------------------------
# The pages say nothing of NaN or infinity.  The rule taken (both sides): a
# NaN encodes as code 0 (E2M1 +0, E4M3 0, INT8 0) and never enters an amax;
# a row (INT8) or tensor (NVFP4) holding an infinity has an infinite amax,
# which makes every reciprocal zero, so its scale is +inf and its codes 0.
# The pins below are consequences that hold for any implementation of that
# rule and fail for the plausible alternatives (NaN saturating to +-127 or
# +-6, a NaN amax, a sign-keeping NaN code).

_QNAN, _NQNAN, _SNAN = 0x7FC0, 0xFFC0, 0x7F81    # bf16 NaN patterns
_PINF, _NINF = 0x7F80, 0xFF80


def test_codecs_encode_nan_as_zero(orc):
    for v in (float("nan"), -float("nan")):
        assert orc.e2m1_encode(v) == 0
        assert orc.e4m3_encode(v) == 0
    assert orc.e2m1_encode(float("inf")) == 7 and orc.e2m1_encode(-float("inf")) == 15
    assert orc.e4m3_encode(float("inf")) == 0x7E


@pytest.mark.parametrize("nan", [_QNAN, _NQNAN, _SNAN])
def test_int8_nan_element_is_a_zero(orc, nan):
    """Without the Hadamard a NaN element codes 0 and the rest of its row
    quantizes as if the NaN were 0 (it never sets the amax)."""
    rng = np.random.default_rng(11)
    x = workloads.activations(rng, 6, 64)
    z = x.copy()
    x[2, 5] = nan
    z[2, 5] = 0
    x[4, 63] = nan
    z[4, 63] = 0
    a = orc.quant_int8(x, flags=orc.NO_HADAMARD)
    b = orc.quant_int8(z, flags=orc.NO_HADAMARD)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_int8_nan_spreads_over_its_hadamard_block(orc):
    """With the Hadamard every output of a block depends on every input, so a
    NaN makes the whole rotated block NaN: the row quantizes as if that block
    were zero."""
    rng = np.random.default_rng(12)
    x = workloads.activations(rng, 4, 96)
    z = x.copy()
    x[1, 37] = _QNAN          # block 2 of row 1
    z[1, 32:48] = 0
    x[3, 0] = _NINF           # with one infinity per block every output is +-inf...
    x[3, 1] = _PINF           # ... with two, some are inf - inf = NaN
    a = orc.quant_int8(x)
    b = orc.quant_int8(z)
    assert np.array_equal(a[0][:3], b[0][:3]) and np.array_equal(a[1][:3], b[1][:3])
    assert np.isinf(a[1][3]) and a[1][3] > 0 and not a[0][3].any()


def test_int8_infinite_row(orc):
    x = np.full((3, 32), 0x3F80, np.uint16)            # 1.0
    x[1, 9] = _PINF
    x[2, 31] = _NINF
    q, s = orc.quant_int8(x, flags=orc.NO_HADAMARD)
    assert s[0] == np.float32(1) / np.float32(127) and np.all(q[0] == 127)
    for r in (1, 2):
        assert s[r] == np.inf and not q[r].any()


@pytest.mark.parametrize("flags", [0, 1])
def test_nvfp4_nan_element_is_a_zero(orc, flags):
    """A NaN never sets the tensor or block amax and codes +0.  Without the
    Hadamard only its own code changes; with it, its whole block quantizes as a
    zero block (scale 0, codes 0)."""
    rng = np.random.default_rng(13)
    x = workloads.activations(rng, 8, 64)
    z = x.copy()
    x[3, 21] = _NQNAN
    x[6, 0] = _SNAN
    if flags:
        z[3, 21] = z[6, 0] = 0
    else:
        z[3, 16:32] = z[6, 0:16] = 0
    a = orc.quant_nvfp4(x, flags=flags)
    b = orc.quant_nvfp4(z, flags=flags)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


@pytest.mark.parametrize("inf", [_PINF, _NINF])
def test_nvfp4_infinite_tensor(orc, inf):
    rng = np.random.default_rng(14)
    x = workloads.activations(rng, 5, 48)
    x[4, 40] = inf
    for flags in (0, 1):
        c, s, g = orc.quant_nvfp4(x, flags=flags)
        assert g == np.inf and not c.any() and not s.any()


def test_w8_from_infinite_tensor_scale(orc):
    """An NVFP4 weight with an infinite tensor scale: every nonzero code
    dequantizes to +-inf and every zero code to 0 * inf = NaN, so each row with
    a nonzero code gets scale +inf; every code is 0."""
    rng = np.random.default_rng(15)
    N, K = 4, 32
    cw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    cw[3] = 0
    sw = rng.integers(1, 0x7F, (N, K // 16)).astype(np.uint8)
    q, s = orc.w8_from_nvfp4(cw, sw, np.float32(np.inf))
    assert np.all(s[:3] == np.inf) and not q.any()
    assert s[3] == 0               # all NaN: the amax stays 0, a zero row
