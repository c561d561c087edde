"""GPU parity of the Purified Delta Refresh pieces against the oracle.

* Outlier count (|x| above kappa times the token row's RMS, decided as
  x^2 K > kappa^2 sum x^2 in fp64): the count is an integer, but the row sums
  are added in a different order on the two sides, so the GPU count must lie
  in the oracle's band [count above threshold*(1+1e-12), count above
  threshold*(1-1e-12)]; for these inputs the band is a single value and the
  counts are equal.
* PDR decision: identical to the oracle's on the same count.
* BF16 GEMM: |y - y_ref| <= 1e-5 * B with B = sum_k |x_k w_k| (exact bf16
  products, fp32 accumulation in a free order), bf16 output within
  1e-5 B + 2^-8 |y_ref|; shapes with a partial last stage (K % 64 != 0) too.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, empty, host, require_gpu, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _count(x_bits, kappa):
    M, K = x_bits.shape
    out = torch.zeros(1, dtype=torch.float64, device="cuda")
    dm.outlier_count(dev(x_bits).view(M, K), kappa, out, dm.new_workspace(dm.OP_OUTLIER))
    torch.cuda.synchronize()
    return float(host(out)[0])


def _check_count(orc, x_bits, kappa):
    c = _count(x_bits, kappa)
    lo, hi = orc.outlier_count_band(x_bits, kappa, 1e-12)
    assert c == int(c) and lo <= c <= hi, (c, lo, hi)
    if lo == hi:
        assert c == orc.outlier_count(x_bits, kappa)
    return c


@pytest.mark.parametrize("M,K", [(1, 16), (7, 48), (300, 1920), (50, 12288), (3, 32768),
                                 (workloads.M_480P, 3072)])
@pytest.mark.parametrize("kappa", [3.0, 6.0])
def test_outlier_count_parity(orc, M, K, kappa):
    require_gpu()
    say(f"outlier_count M={M} K={K} kappa={kappa}")
    x = workloads.activations(np.random.default_rng(M + K), M, K)
    c = _check_count(orc, x, kappa)
    if M * K > 4096:
        assert 0 < c < M * K


def test_outlier_count_edges(orc):
    require_gpu()
    say("outlier_count edge cases")
    z = np.zeros((5, 64), np.uint16)
    assert _check_count(orc, z, 2.0) == 0
    rng = np.random.default_rng(7)
    x = workloads.activations(rng, 9, 80)
    assert _check_count(orc, x, 0.0) == np.count_nonzero(workloads.bf16_bits_to_f32(x))
    spike = np.zeros((4, 64), np.float32)
    spike[:, 3] = [1.0, -2.0, 1e-30, 3e30]
    sb = workloads.to_bf16_bits(spike)
    assert _check_count(orc, sb, 7.95) == 4 and _check_count(orc, sb, 8.0) == 0
    # the count compares magnitude bits with a per-row threshold: rows with an
    # infinity or a NaN count nothing (their sum of squares is not finite),
    # the other rows count as usual; subnormal and near-maximal magnitudes
    rng = np.random.default_rng(11)
    sp = workloads.activations(rng, 8, 64)
    sp[0, 5], sp[1, 0], sp[2, 63], sp[3, 7] = 0x7F80, 0xFF80, 0x7FC0, 0xFFC1
    sp[4] = rng.integers(0, 0x80, 64).astype(np.uint16) | (rng.integers(0, 2, 64).astype(np.uint16) << 15)
    sp[4, 9] = 0x0070                                  # a subnormal spike
    sp[5] = 0x7F7F                                     # the largest finite bf16, every element
    sp[6, :] = 0x0001
    sp[6, 3] = 0x0100                                  # the smallest subnormal, one normal spike
    for kappa in (0.0, 1.0, 3.0, 7.9):
        c = _check_count(orc, sp, kappa)
        per_row = [orc.outlier_count(sp[r:r + 1], kappa) for r in range(8)]
        assert per_row[:4] == [0, 0, 0, 0] and c == sum(per_row)
    assert _check_count(orc, sp[6:7], 7.9) == 1 and _check_count(orc, sp[5:6], 0.5) == 64
    out = torch.full((1,), 7.0, dtype=torch.float64, device="cuda")
    dm.outlier_count(torch.empty((0, 64), dtype=torch.int16, device="cuda"), 2.0, out,
                     dm.new_workspace(dm.OP_OUTLIER))
    torch.cuda.synchronize()
    assert float(host(out)[0]) == 0.0


def test_pdr_decide_matches_oracle(orc):
    require_gpu()
    for count, n, rho in [(11, 100, 0.1), (10, 100, 0.1), (0, 100, 0.0), (1, 100, 0.0), (0, 0, 0.0),
                          (5, 1_000_000, 1e-6), (4, 1_000_000, 4e-6)]:
        assert dm.pdr_decide(count, n, rho) == orc.pdr_force(count, n, rho)


def _gemm(x_bits, w_bits, out_dtype):
    M, K = x_bits.shape
    N = w_bits.shape[0]
    y = empty((M, N), np.float32 if out_dtype == dm.OUT_F32 else np.uint16)
    dm.gemm_bf16(dev(x_bits).view(M, K), dev(w_bits).view(N, K), y, out_dtype)
    torch.cuda.synchronize()
    return y


def _check_gemm(orc, x, w, rows=None):
    y0, b0 = orc.gemm_bf16(x, w, rows=rows)
    sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
    y1 = host(_gemm(x, w, dm.OUT_F32)[sel]).astype(np.float64)
    err = np.abs(y1 - y0)
    assert np.all(err <= TOL * b0), float((err / np.maximum(b0, 1e-300)).max())
    yb = workloads.bf16_bits_to_f32(host(_gemm(x, w, dm.OUT_BF16)[sel], np.uint16)).astype(np.float64)
    assert np.all(np.abs(yb - y0) <= TOL * b0 + 2.0 ** -8 * np.abs(y0))


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (256, 256, 64), (200, 136, 80), (129, 257, 384),
                                   (64, 96, 1920), (33, 40, 12288), (300, 130, 48), (513, 300, 1008)])
def test_gemm_bf16_parity(orc, M, N, K):
    require_gpu()
    say(f"gemm_bf16 M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 13 * N + K)
    _check_gemm(orc, workloads.activations(rng, M, K), workloads.weight(rng, N, K))


def test_gemm_bf16_empty():
    require_gpu()
    dm.gemm_bf16(empty((0, 32), np.uint16), empty((8, 32), np.uint16), empty((0, 8), np.float32))
    dm.gemm_bf16(empty((4, 32), np.uint16), empty((0, 32), np.uint16), empty((4, 0), np.float32))
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K", [(workloads.M_480P, 9216, 3072), (workloads.M_480P, 3072, 12288),
                                   (workloads.M_480P, 5760, 1920)])
def test_gemm_bf16_full_shape_sampled(orc, M, N, K):
    require_gpu()
    say(f"gemm_bf16 full M={M} N={N} K={K} (row sample)")
    rng = np.random.default_rng(N + 2 * K)
    rows = np.unique(np.concatenate([np.arange(0, M, 211), np.arange(M - 3, M)]))
    _check_gemm(orc, workloads.activations(rng, M, K), workloads.weight(rng, N, K), rows=rows)
