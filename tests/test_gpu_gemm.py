"""GPU parity: INT8 and NVFP4 quantized GEMMs against the oracle.

INT8: int32 accumulators and the fp32 epilogue bit-exact (and bf16 output =
RNE of that fp32).  NVFP4 (both variants: 16-bit dequant + MFMA, and the
block-scaled f8f6f4 MFMA with fp32 rescale): per element |y - y_ref| <=
1e-5 * B with B = gA gW sum_k |a_k||w_k| (the fp32 summation scale), since
only the fp32 accumulation order is free.  Full CogVideoX-like shapes are checked on a
deterministic row sample (every 211th row plus the last 3 rows).
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, empty, host, require_gpu, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _quantized_pair(orc, rng, M, N, K):
    x = workloads.activations(rng, M, K)
    w = workloads.weight(rng, N, K)
    return orc.quant_int8(x), orc.quant_nvfp4(x), orc.prep_weight(w)


def _rows(M):
    return np.unique(np.concatenate([np.arange(0, M, 211), np.arange(max(M - 3, 0), M)]))


def _run_int8(qa, sa, qw, sw, out_dtype):
    M, K = qa.shape
    N = qw.shape[0]
    y = empty((M, N), {dm.OUT_F32: np.float32, dm.OUT_BF16: np.uint16, dm.OUT_I32: np.int32}[out_dtype])
    dm.qgemm_int8(dev(qa), dev(sa), dev(qw), dev(sw), y, out_dtype)
    torch.cuda.synchronize()
    return y


def _run_nvfp4(ca, sa, ga, cw, sw, gw, out_dtype=dm.OUT_F32, variant=dm.FP4_BF16_DEQUANT):
    M, N = ca.shape[0], cw.shape[0]
    y = empty((M, N), np.float32 if out_dtype == dm.OUT_F32 else np.uint16)
    dm.qgemm_nvfp4(dev(ca), dev(sa), dev(np.array([ga], np.float32)), dev(cw), dev(sw),
                   dev(np.array([gw], np.float32)), y, out_dtype, variant)
    torch.cuda.synchronize()
    return y


def _check_int8(orc, qa, sa, qw, sw, rows=None):
    acc0, y0 = orc.gemm_int8(qa, sa, qw, sw, rows=rows)
    sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
    acc1 = host(_run_int8(qa, sa, qw, sw, dm.OUT_I32)[sel])
    assert np.array_equal(acc1, acc0)
    y1 = host(_run_int8(qa, sa, qw, sw, dm.OUT_F32)[sel])
    assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32))
    yb = host(_run_int8(qa, sa, qw, sw, dm.OUT_BF16)[sel], np.uint16)
    assert np.array_equal(yb, workloads.to_bf16_bits(y0))


FP4_VARIANTS = (dm.FP4_BF16_DEQUANT, dm.FP4_SCALED_MFMA)


def _check_nvfp4(orc, ca, sa, ga, cw, sw, gw, rows=None, variants=FP4_VARIANTS):
    """Both GEMM variants against one oracle evaluation."""
    y0, b0 = orc.gemm_nvfp4(ca, sa, ga, cw, sw, gw, rows=rows)
    sel = slice(None) if rows is None else torch.from_numpy(rows).cuda()
    for v in variants:
        y1 = host(_run_nvfp4(ca, sa, ga, cw, sw, gw, variant=v)[sel]).astype(np.float64)
        err = np.abs(y1 - y0)
        assert np.all(err <= TOL * b0), (v, float((err / np.maximum(b0, 1e-300)).max()))
        # report-style check: typical relative error is far below the bound
        big = np.abs(y0) > 1e-3 * b0
        if big.any():
            assert np.median(err[big] / np.abs(y0[big])) < 1e-5, v
        yb = host(_run_nvfp4(ca, sa, ga, cw, sw, gw, dm.OUT_BF16, v)[sel], np.uint16)
        ybf = workloads.bf16_bits_to_f32(yb).astype(np.float64)
        assert np.all(np.abs(ybf - y0) <= TOL * b0 + 2.0 ** -8 * np.abs(y0)), v


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (256, 256, 256), (200, 136, 80), (129, 257, 384),
                                   (64, 96, 1920), (33, 40, 12288), (300, 130, 48)])
def test_int8_gemm_parity(orc, M, N, K):
    require_gpu()
    say(f"qgemm_int8 M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 3 * N + 5 * K)
    (qa, sa), _, p = _quantized_pair(orc, rng, M, N, K)
    _check_int8(orc, qa, sa, p["qw"], p["sw_row"])


def test_int8_gemm_extremes(orc):
    # every operand at +-127, K = 12288: the largest int32 accumulators
    require_gpu()
    say("qgemm_int8 extremes")
    M, N, K = 70, 65, 12288
    qa = np.full((M, K), 127, np.int8)
    qa[1::2] = -127
    qw = np.full((N, K), -127, np.int8)
    sa = np.ones(M, np.float32)
    sw = np.full(N, 0.5, np.float32)
    _check_int8(orc, qa, sa, qw, sw)


# K % 256 == 128 from 384 closes with a half stage (384, 640, 1152, 1920, 2432);
# K = 128 takes the K % 64 kernel
@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (256, 256, 256), (200, 136, 80), (129, 257, 384),
                                   (64, 96, 1920), (33, 40, 12288), (300, 130, 48), (1, 1, 256),
                                   (129, 257, 512), (513, 300, 768), (257, 130, 640), (70, 520, 1152),
                                   (300, 300, 2432), (129, 70, 128)])
def test_nvfp4_gemm_parity(orc, M, N, K):
    require_gpu()
    say(f"qgemm_nvfp4 M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 7 * N + 11 * K)
    _, (ca, sa, ga), p = _quantized_pair(orc, rng, M, N, K)
    _check_nvfp4(orc, ca, sa, ga, p["cw"], p["sw"], p["gw"])


def test_nvfp4_gemm_random_codes(orc):
    # arbitrary codes and scales (all 16 E2M1 codes, all finite E4M3 scales)
    require_gpu()
    say("qgemm_nvfp4 random codes")
    rng = np.random.default_rng(70)
    M, N, K = 150, 140, 320
    ca = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    cw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sa = rng.integers(0, 0x7F, (M, K // 16)).astype(np.uint8)
    sw = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    _check_nvfp4(orc, ca, sa, 0.75, cw, sw, 1.5e-3)
    _check_nvfp4(orc, ca, sa, 0.0, cw, sw, 1.0)
    for K in (512, 640):  # 256-element stages; and two with the closing half stage
        ca = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
        cw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
        sa = rng.integers(0, 0x7F, (M, K // 16)).astype(np.uint8)
        sw = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
        _check_nvfp4(orc, ca, sa, 0.75, cw, sw, 1.5e-3)


def test_gemm_max_k(orc):
    """K = 2^22, the largest K the GEMM entry points take (the DMA kernels
    address 256 rows from a scalar base by 32-bit offsets): INT8, NVFP4 and
    BF16 against the oracle on a few rows and columns."""
    require_gpu()
    M, N, K = 3, 5, 1 << 22
    say(f"GEMMs at the largest K: M={M} N={N} K={K}")
    rng = np.random.default_rng(22)
    (qa, sa), (ca, sca, ga), p = _quantized_pair(orc, rng, M, N, K)
    _check_int8(orc, qa, sa, p["qw"], p["sw_row"])
    _check_nvfp4(orc, ca, sca, ga, p["cw"], p["sw"], p["gw"], variants=(dm.FP4_BF16_DEQUANT,))
    x, w = workloads.activations(rng, M, K), workloads.weight(rng, N, K)
    y0, b0 = orc.gemm_bf16(x, w)
    y = empty((M, N), np.float32)
    dm.gemm_bf16(dev(x), dev(w), y)
    torch.cuda.synchronize()
    assert np.all(np.abs(host(y).astype(np.float64) - y0) <= TOL * b0)


def test_gemm_empty():
    require_gpu()
    say("qgemm empty shapes")
    y = empty((0, 8), np.float32)
    dm.qgemm_int8(empty((0, 32), np.int8), empty((0,), np.float32), empty((8, 32), np.int8),
                  empty((8,), np.float32), y)
    y2 = empty((4, 0), np.float32)
    for v in FP4_VARIANTS:
        dm.qgemm_nvfp4(empty((4, 16), np.uint8), empty((4, 2), np.uint8), torch.ones(1, device="cuda"),
                       empty((0, 16), np.uint8), empty((0, 2), np.uint8), torch.ones(1, device="cuda"),
                       y2, dm.OUT_F32, v)
    torch.cuda.synchronize()


FULL = [(workloads.M_480P, 9216, 3072), (workloads.M_480P, 3072, 12288),
        (workloads.M_480P, 5760, 1920)]


@pytest.mark.parametrize("M,N,K", FULL)
def test_int8_gemm_full_shape_sampled(orc, M, N, K):
    require_gpu()
    say(f"qgemm_int8 full M={M} N={N} K={K} (row sample)")
    rng = np.random.default_rng(N + K)
    (qa, sa), _, p = _quantized_pair(orc, rng, M, N, K)
    _check_int8(orc, qa, sa, p["qw"], p["sw_row"], rows=_rows(M))


@pytest.mark.parametrize("M,N,K", FULL)
def test_nvfp4_gemm_full_shape_sampled(orc, M, N, K):
    require_gpu()
    say(f"qgemm_nvfp4 full M={M} N={N} K={K} (row sample)")
    rng = np.random.default_rng(N + K + 1)
    _, (ca, sa, ga), p = _quantized_pair(orc, rng, M, N, K)
    _check_nvfp4(orc, ca, sa, ga, p["cw"], p["sw"], p["gw"], rows=_rows(M))
