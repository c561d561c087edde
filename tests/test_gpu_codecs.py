"""GPU converters against the oracle's encoders on every finite fp32 input.

The quantizers encode block scales with the library's E4M3 encoder and
elements with the chip's E2M1 converter.  Both are monotone step functions
of the input's bit pattern (E2M1 of a negative input mirrors the positive
one, with the sign bit).  The library's self-test reports, per output code,
the lowest and highest input pattern that produce it and how many do; the
same three numbers follow from the oracle's nearest-value encoders by
bisection over the patterns.  Equal numbers for every code mean equal
outputs for all 2^31 - 2^23 finite non-negative patterns (and their
negatives for E2M1), including every midpoint and its neighbours.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
from gpu_util import host, require_gpu, say

pytestmark = pytest.mark.gpu

FINITE = 0x7F800000  # +inf: patterns below it are the finite non-negative floats


def _f(p: int) -> float:
    return float(np.array([p], np.uint32).view(np.float32)[0])


def _runs(encode, lo: int, hi: int, ncodes: int) -> np.ndarray:
    """Per code (lowest, highest, count) of the patterns [lo, hi), for an
    encoder that is non-decreasing in the pattern."""
    st = np.zeros((ncodes, 3), np.uint64)
    st[:, 0] = 0xFFFFFFFF
    a = lo
    while a < hi:
        c = encode(a)
        lo_b, hi_b = a, hi          # first pattern past a with another code lies in (lo_b, hi_b]
        while hi_b - lo_b > 1:
            mid = (lo_b + hi_b) // 2
            if encode(mid) == c:
                lo_b = mid
            else:
                hi_b = mid
        st[c] = (a, hi_b - 1, hi_b - a)
        a = hi_b
    return st


def _gpu(codec: int, lo: int, hi: int, rows: int) -> np.ndarray:
    stats = torch.zeros(3 * rows, dtype=torch.int32, device="cuda")
    dm.selftest_codec(codec, lo, hi, stats)
    torch.cuda.synchronize()
    return host(stats, np.uint32).reshape(rows, 3).astype(np.uint64)


def test_e4m3_encoder_every_input(orc):
    require_gpu()
    say("E4M3 encoder over every finite non-negative fp32")
    want = _runs(lambda p: orc.e4m3_encode(_f(p)), 0, FINITE, 128)
    got = _gpu(dm.CODEC_E4M3, 0, FINITE, 128)
    assert np.array_equal(got, want), np.nonzero((got != want).any(axis=1))[0]
    assert want[:, 2].sum() == FINITE and want[0x7F, 2] == 0   # 0x7F (NaN) is never produced


def test_e2m1_converter_every_input(orc):
    require_gpu()
    say("E2M1 converter over every finite fp32 of both signs")
    pos = _runs(lambda p: orc.e2m1_encode(_f(p)), 0, FINITE, 16)
    neg = _runs(lambda p: orc.e2m1_encode(-_f(p)) - 8, 0, FINITE, 16)
    want = pos.copy()
    want[8:16] = neg[0:8]
    got = _gpu(dm.CODEC_E2M1, 0, FINITE, 16)
    assert np.array_equal(got, want), np.nonzero((got != want).any(axis=1))[0]
    assert want[:8, 2].sum() == FINITE and want[8:, 2].sum() == FINITE


def test_codec_subrange(orc):
    """A range that starts and ends inside runs (the chunk edges of the
    kernel's walk fall elsewhere than for the full range)."""
    require_gpu()
    lo, hi = 0x3E7FFF00, 0x40C00123   # about 0.25 .. 6.0000x
    for codec, rows, enc in ((dm.CODEC_E4M3, 128, lambda p: orc.e4m3_encode(_f(p))),
                             (dm.CODEC_E2M1, 16, lambda p: orc.e2m1_encode(_f(p)))):
        want = _runs(enc, lo, hi, rows)
        got = _gpu(codec, lo, hi, rows)
        if codec == dm.CODEC_E2M1:
            assert np.array_equal(got[:8], want[:8])
        else:
            assert np.array_equal(got, want)
