"""GPU parity: the INT8 GEMM that converts its NVFP4 weight inside the
weight-tile load (dmpq_qgemm_int8_from_nvfp4).

Its B operand is the NVFP4 weight requantized to INT8 by the rule of
dmpq_weight_int8_from_nvfp4, computed by the same operations in the same
order, so its output must equal the chain "convert, then INT8 GEMM" bit for
bit: int32 accumulators, fp32 and bf16 outputs, GELU and the fused amax.  One
shape is also checked straight against the oracle's conversion and INT8
GEMM, and the non-finite tensor scales of the conversion's rule (0, inf,
NaN) are covered, as is a weight row of zero codes.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, empty, host, require_gpu, say

pytestmark = pytest.mark.gpu

_OUT_NP = {dm.OUT_F32: np.float32, dm.OUT_BF16: np.uint16, dm.OUT_I32: np.int32}


def _inputs(orc, rng, M, N, K):
    qa, sa = orc.quant_int8(workloads.activations(rng, M, K))
    p = orc.prep_weight(workloads.weight(rng, N, K))
    return qa, sa, p["cw"], p["sw"], p["gw"]


def _fused(qa, sa, cw, sw, gw, out_dtype, epilogue=0):
    M, N = qa.shape[0], cw.shape[0]
    y = empty((M, N), _OUT_NP[out_dtype])
    ws = dm.new_workspace(dm.OP_GEMM_W4, "cuda", M, N)
    dm.qgemm_int8_from_nvfp4(dev(qa), dev(sa), dev(cw), dev(sw), dev(np.array([gw], np.float32)), y, ws,
                             epilogue, out_dtype)
    torch.cuda.synchronize()
    return y, ws


def _chain(qa, sa, cw, sw, gw, out_dtype, epilogue=0):
    M, K = qa.shape
    N = cw.shape[0]
    qw = empty((N, K), np.int8)
    sw_row = empty((N,), np.float32)
    dm.weight_int8_from_nvfp4(dev(cw), dev(sw), dev(np.array([gw], np.float32)), qw, sw_row)
    y = empty((M, N), _OUT_NP[out_dtype])
    ws = dm.new_workspace(dm.OP_GEMM_AMAX, "cuda", M, N) if epilogue & dm.EPI_NVFP4_AMAX else None
    dm.qgemm_int8_ex(dev(qa), dev(sa), qw, sw_row, y, epilogue, ws, out_dtype)
    torch.cuda.synchronize()
    return y, ws


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (256, 256, 256), (200, 136, 384), (300, 528, 512),
                                   (64, 96, 1920), (33, 40, 12288), (513, 300, 3072)])
def test_fused_equals_convert_then_gemm(orc, M, N, K):
    require_gpu()
    say(f"qgemm_int8_from_nvfp4 M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 5 * N + 9 * K)
    qa, sa, cw, sw, gw = _inputs(orc, rng, M, N, K)
    for od in (dm.OUT_I32, dm.OUT_F32, dm.OUT_BF16):
        assert _same(_fused(qa, sa, cw, sw, gw, od)[0], _chain(qa, sa, cw, sw, gw, od)[0]), od


def test_fused_against_oracle(orc):
    require_gpu()
    say("qgemm_int8_from_nvfp4 against the oracle")
    rng = np.random.default_rng(44)
    M, N, K = 290, 270, 640
    qa, sa, cw, sw, gw = _inputs(orc, rng, M, N, K)
    qw, sw_row = orc.w8_from_nvfp4(cw, sw, gw)
    acc0, y0 = orc.gemm_int8(qa, sa, qw, sw_row)
    assert np.array_equal(host(_fused(qa, sa, cw, sw, gw, dm.OUT_I32)[0]), acc0)
    y1 = host(_fused(qa, sa, cw, sw, gw, dm.OUT_F32)[0])
    assert np.array_equal(y1.view(np.uint32), y0.view(np.uint32))


@pytest.mark.parametrize("epilogue", [dm.EPI_GELU, dm.EPI_NVFP4_AMAX, dm.EPI_GELU | dm.EPI_NVFP4_AMAX])
def test_fused_epilogues(orc, epilogue):
    require_gpu()
    say(f"qgemm_int8_from_nvfp4 epilogue {epilogue}")
    rng = np.random.default_rng(epilogue + 60)
    M, N, K = 300, 528, 512
    qa, sa, cw, sw, gw = _inputs(orc, rng, M, N, K)
    ya, wa = _fused(qa, sa, cw, sw, gw, dm.OUT_BF16, epilogue)
    yb, wb = _chain(qa, sa, cw, sw, gw, dm.OUT_BF16, epilogue)
    assert _same(ya, yb)
    if epilogue & dm.EPI_NVFP4_AMAX:
        tiles = ((M + 255) // 256) * ((N + 255) // 256)
        assert torch.equal(wa[:4 * tiles], wb[:4 * tiles])


@pytest.mark.parametrize("gw", [0.0, float("inf"), float("nan"), 3.0e38])
def test_fused_tensor_scale_edges(orc, gw):
    # zero, infinite and NaN tensor scales, and one whose products overflow,
    # follow the conversion's rule (zero rows store zeros; an infinite amax
    # gives scale +inf); a weight row of zero codes is a zero row
    require_gpu()
    say(f"qgemm_int8_from_nvfp4 tensor scale {gw}")
    rng = np.random.default_rng(7)
    M, N, K = 130, 140, 256
    qa, sa, cw, sw, _ = _inputs(orc, rng, M, N, K)
    cw = cw.copy()
    cw[3] = 0
    for od in (dm.OUT_I32, dm.OUT_F32):
        assert _same(_fused(qa, sa, cw, sw, gw, od)[0], _chain(qa, sa, cw, sw, gw, od)[0]), od


@pytest.mark.parametrize("M,N,K", [(workloads.M_480P, 9216, 3072), (workloads.M_480P, 3072, 12288)])
def test_fused_full_shape(orc, M, N, K):
    require_gpu()
    say(f"qgemm_int8_from_nvfp4 full M={M} N={N} K={K}")
    rng = np.random.default_rng(N + K + 8)
    qa, sa, cw, sw, gw = _inputs(orc, rng, M, N, K)
    assert _same(_fused(qa, sa, cw, sw, gw, dm.OUT_BF16)[0], _chain(qa, sa, cw, sw, gw, dm.OUT_BF16)[0])


def test_fused_errors_and_empty():
    require_gpu()
    say("qgemm_int8_from_nvfp4 errors and empty shapes")
    one = torch.ones(1, device="cuda")
    M, N = 4, 8
    y = empty((M, N), np.float32)
    with pytest.raises(dm.DmpqError) as e:  # K % 128 != 0
        dm.qgemm_int8_from_nvfp4(empty((M, 64), np.int8), empty((M,), np.float32), empty((N, 32), np.uint8),
                                 empty((N, 4), np.uint8), one, y, dm.new_workspace(dm.OP_GEMM_W4, "cuda", M, N),
                                 0, dm.OUT_F32)
    assert e.value.status == 4  # DMPQ_ERR_UNSUPPORTED
    small = torch.zeros(dm.workspace_bytes(dm.OP_GEMM_W4, M, N) - 4, dtype=torch.uint8, device="cuda")
    for ws in (None, small):
        with pytest.raises(dm.DmpqError) as e:
            dm.qgemm_int8_from_nvfp4(empty((M, 128), np.int8), empty((M,), np.float32),
                                     empty((N, 64), np.uint8), empty((N, 8), np.uint8), one, y, ws, 0, dm.OUT_F32)
        assert e.value.status == 6  # DMPQ_ERR_WORKSPACE
    dm.qgemm_int8_from_nvfp4(empty((0, 128), np.int8), empty((0,), np.float32), empty((N, 64), np.uint8),
                             empty((N, 8), np.uint8), one, empty((0, N), np.float32),
                             dm.new_workspace(dm.OP_GEMM_W4, "cuda", 0, N), 0, dm.OUT_F32)
    torch.cuda.synchronize()
