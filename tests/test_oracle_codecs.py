"""Pins for the oracle's number codecs (bf16, E2M1, E4M3).

Pinned against: the OCP format tables in tests/golden (published specs),
exhaustive decode->encode identity, every midpoint between neighbouring
codes (ties to the even code) and one ulp either side, saturation, and
torch's own bf16 conversion (an independent implementation).
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 0), float(v)))
    return rows


def _f32(x):
    return float(np.float32(x))


def _up(x):
    return float(np.nextafter(np.float32(x), np.float32(np.inf)))


def _down(x):
    return float(np.nextafter(np.float32(x), np.float32(-np.inf)))


# ---- E2M1 -----------------------------------------------------------------

def test_e2m1_decode_matches_ocp_table(orc):
    table = _read_table("e2m1_values.txt")
    assert len(table) == 8
    for code, val in table:
        assert orc.e2m1_value(code) == val
        neg = orc.e2m1_value(code | 8)
        assert neg == -val and math.copysign(1.0, neg) == -1.0


def test_e2m1_roundtrip_all_codes(orc):
    for code in range(16):
        assert orc.e2m1_encode(orc.e2m1_value(code)) == code


def test_e2m1_midpoints_tie_to_even(orc):
    mags = [orc.e2m1_value(c) for c in range(8)]
    for c in range(7):
        mid = (mags[c] + mags[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert orc.e2m1_encode(mid) == even, (c, mid)
        assert orc.e2m1_encode(_down(mid)) == c
        assert orc.e2m1_encode(_up(mid)) == c + 1
        assert orc.e2m1_encode(-mid) == 8 | even


def test_e2m1_saturates_and_keeps_zero_sign(orc):
    for v in (6.0, _up(6.0), 6.5, 7.0, 100.0, 3.0e38):
        assert orc.e2m1_encode(v) == 7
        assert orc.e2m1_encode(-v) == 15
    assert orc.e2m1_encode(0.0) == 0
    assert orc.e2m1_encode(-0.0) == 8
    assert orc.e2m1_encode(-0.1) == 8      # rounds to zero, keeps the sign
    assert orc.e2m1_encode(1e-30) == 0


def test_e2m1_nearest_by_brute_force(orc):
    rng = np.random.default_rng(0)
    mags = np.array([orc.e2m1_value(c) for c in range(8)])
    for v in rng.uniform(0, 7, 2000).astype(np.float32):
        d = np.abs(mags - float(v))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert orc.e2m1_encode(float(v)) == want


# ---- E4M3 -----------------------------------------------------------------

def test_e4m3_anchor_values(orc):
    for code, val in _read_table("e4m3_anchor_values.txt"):
        got = orc.e4m3_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_e4m3_decode_formula_all_codes(orc):
    # independent restatement of the format: bias 7, 3 mantissa bits, subnormals at e=0
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        want = math.ldexp(m, -9) if e == 0 else math.ldexp(1 + m / 8, e - 7)
        assert orc.e4m3_value(code) == want


def test_e4m3_roundtrip_and_monotone(orc):
    vals = [orc.e4m3_value(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))
    for c in range(0x7F):
        assert orc.e4m3_encode(vals[c]) == c


def test_e4m3_midpoints_tie_to_even(orc):
    vals = [orc.e4m3_value(c) for c in range(0x7F)]
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2
        assert _f32(mid) == mid
        even = c if c % 2 == 0 else c + 1
        assert orc.e4m3_encode(mid) == even, hex(c)
        assert orc.e4m3_encode(_down(mid)) == c
        assert orc.e4m3_encode(_up(mid)) == c + 1


def test_e4m3_saturation_and_underflow(orc):
    for v in (448.0, _up(448.0), 464.0, 480.0, 1e6, 3e38):
        assert orc.e4m3_encode(v) == 0x7E
    assert orc.e4m3_encode(0.0) == 0
    assert orc.e4m3_encode(2.0 ** -10) == 0          # tie between 0 and 2^-9 -> even (0)
    assert orc.e4m3_encode(_up(2.0 ** -10)) == 1
    assert orc.e4m3_encode(1e-20) == 0


# ---- bf16 -----------------------------------------------------------------

def test_bf16_roundtrip_all_patterns(orc):
    for b in range(1 << 16):
        v = orc.bf16_value(b)
        if math.isnan(v):
            assert orc.bf16_round(v) == 0x7FC0
            continue
        assert orc.bf16_round(v) == b


@pytest.mark.parametrize("seed", [0, 1])
def test_bf16_round_matches_torch(orc, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, 4000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # also exact ties: bf16 value + half an ulp
    base = rng.integers(0, 2**15, 1000, dtype=np.uint32) << 16 | 0x8000
    vals = np.concatenate([vals, base.view(np.float32)])
    vals = vals[np.isfinite(vals)]
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_round(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, want)
