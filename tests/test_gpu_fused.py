"""GPU checks of the producer-fused epilogues of the three linears.

GELU (DMPQ_EPI_GELU): the output must be bf16(GELU(bf16(v))) for the
linear's value v.  INT8 values are bit-exact, so the pre-activation is the
oracle's bf16 value exactly and only GELU's own fp32 evaluation and the
final rounding are free: every element within that bound, and at least 99%
identical to bf16 of the oracle's fp64 GELU.  For the NVFP4 and BF16
linears the pre-activation carries the GEMM tolerance (1e-5 * B, B the
summation scale), propagated through GELU's Lipschitz constant (1.129).

Fused NVFP4 amax (DMPQ_EPI_NVFP4_AMAX): the per-tile maxima the kernel
leaves in the workspace equal, as a multiset, max |H16 rotation| of each
256 x 256 tile of the stored output, recomputed on the host in the same fp32
butterfly order; the quantizer's given-amax mode then produces exactly the
bits of its own two-pass mode on that output.  Shapes span several tiles
with ragged row and column tails and every main-loop path of each GEMM; the
largest output is planted in the last (ragged) tile, in the first, or spread.
"""
import numpy as np
import pytest
import torch
from scipy.special import erfc

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, empty, host, require_gpu, say

pytestmark = pytest.mark.gpu

TOL = 1e-5          # GEMM fp32-accumulation tolerance, relative to B
LIP = 1.13          # max |GELU'(u)| = 1.1289 at u = sqrt 2
HALF_ULP = 2.0 ** -8


def _gelu_rel(v):
    """Relative error bound of the kernel's fp32 GELU: the erfc fit (1.2e-7),
    a few ulp of the reciprocal, exp2 and products, plus the rounding of the
    exponent -v^2/2 + P (about v^2 * 1.2e-7 relative in erfc's tail), with
    a factor of two of margin."""
    return 4e-6 + v * v * 2.5e-7


def _hadamard_tile_max(y_bits, M, N):
    """max |H16 rotation of each 16-block| per 256 x 256 tile, fp32 butterflies
    in stages 1, 2, 4, 8, then * 1/4 (each numpy op rounds to fp32 once)."""
    f = workloads.bf16_bits_to_f32(y_bits).astype(np.float32).reshape(M, N // 16, 16)
    h = 1
    while h < 16:
        idx = np.arange(16)
        lo = idx[(idx & h) == 0]
        a, b = f[:, :, lo].copy(), f[:, :, lo + h].copy()
        f[:, :, lo] = a + b
        f[:, :, lo + h] = a - b
        h *= 2
    r = np.abs(f * np.float32(0.25)).reshape(M, N)
    tm, tn = -(-M // 256), -(-N // 256)
    out = []
    for i in range(tm):
        for j in range(tn):
            out.append(r[256 * i:256 * (i + 1), 256 * j:256 * (j + 1)].max())
    return np.sort(np.array(out, np.float32))


def _plant(x, where):
    """Scale rows of the activation so the largest outputs land in one place."""
    x = workloads.bf16_bits_to_f32(x).copy()
    if where == "last":
        x[-3:] *= 16.0
    elif where == "first":
        x[:2] *= 16.0
    return workloads.to_bf16_bits(x)


def _inputs(orc, kind, M, N, K, seed, where="spread"):
    rng = np.random.default_rng(seed)
    x = _plant(workloads.activations(rng, M, K), where)
    w = workloads.weight(rng, N, K)
    if kind == "bf16":
        return (x, w), None
    if kind == "int8":
        qa, sa = orc.quant_int8(x)
        p = orc.prep_weight(w)
        return (qa, sa, p["qw"], p["sw_row"]), None
    ca, sa, ga = orc.quant_nvfp4(x)
    p = orc.prep_weight(w)
    return (ca, sa, ga, p["cw"], p["sw"], p["gw"]), None


def _reference(orc, kind, args):
    """Oracle pre-activation y0 (fp64 or exact fp32) and its tolerance."""
    if kind == "int8":
        _, y0 = orc.gemm_int8(*args)
        return y0.astype(np.float64), np.zeros(y0.shape)
    if kind == "nvfp4":
        y0, b0 = orc.gemm_nvfp4(*args)
    else:
        y0, b0 = orc.gemm_bf16(*args)
    return y0, TOL * b0


def _run(kind, args, M, N, epilogue, ws):
    y = empty((M, N), np.uint16)
    if kind == "int8":
        qa, sa, qw, sw = args
        dm.qgemm_int8_ex(dev(qa), dev(sa), dev(qw), dev(sw), y, epilogue, ws)
    elif kind == "nvfp4":
        ca, sa, ga, cw, sw, gw = args
        dm.qgemm_nvfp4_ex(dev(ca), dev(sa), dev(np.array([ga], np.float32)), dev(cw), dev(sw),
                          dev(np.array([gw], np.float32)), y, epilogue, ws)
    else:
        x, w = args
        dm.gemm_bf16_ex(dev(x), dev(w), y, epilogue, ws)
    torch.cuda.synchronize()
    return host(y, np.uint16)


# (kind, K): every main loop -- INT8 DMA (K % 128 == 0) and general; NVFP4
# DMA (K % 256, and other K % 128 from 384 with a closing half stage), fast
# (K % 64), 16-bit (K % 16); BF16 with and without tail.
PATHS = [("int8", 256), ("int8", 208), ("nvfp4", 512), ("nvfp4", 384), ("nvfp4", 320), ("nvfp4", 208),
         ("bf16", 256), ("bf16", 208)]


@pytest.mark.parametrize("kind,K", PATHS)
def test_gelu_epilogue(orc, kind, K):
    require_gpu()
    M, N = 600, 528
    say(f"gelu epilogue {kind} M={M} N={N} K={K}")
    args, _ = _inputs(orc, kind, M, N, K, seed=K + len(kind))
    y0, tol0 = _reference(orc, kind, args)
    got = workloads.bf16_bits_to_f32(_run(kind, args, M, N, dm.EPI_GELU, None)).astype(np.float64)
    if kind == "int8":
        pre = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(y0.astype(np.float32)))
        g0 = orc.gelu(pre.astype(np.float64))
        bound = (HALF_ULP + _gelu_rel(pre)) * np.abs(g0) + 1e-30
        assert np.all(np.abs(got - g0) <= bound)
        exact = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(g0.astype(np.float32)))
        assert np.mean(got == exact) >= 0.99
    else:
        g0 = orc.gelu(y0)
        d = tol0 * (1 + HALF_ULP) + HALF_ULP * np.abs(y0)
        bound = LIP * d + (HALF_ULP + _gelu_rel(np.abs(y0) + d)) * (np.abs(g0) + LIP * d) + 1e-30
        err = np.abs(got - g0)
        assert np.all(err <= bound), float((err / bound).max())
    # GELU is not the identity here: large negative values were squashed
    assert y0.min() < -1.0 and got.min() >= -0.1701
    # composition: the fused output is GELU of the plain bf16 output (fp64
    # GELU from scipy here), up to the final rounding of GELU's value
    pre = workloads.bf16_bits_to_f32(_run(kind, args, M, N, 0, None)).astype(np.float64)
    g1 = 0.5 * pre * erfc(-pre / np.sqrt(2.0))
    r1 = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(g1.astype(np.float32)))
    assert np.mean(got == r1) >= 0.99
    assert np.all(np.abs(got - g1) <= (HALF_ULP + _gelu_rel(pre)) * np.abs(g1) + 1e-30)


@pytest.mark.parametrize("kind,K,where", [(k, K, w) for (k, K) in PATHS
                                          for w in ("last", "first", "spread")][::2] +
                         [("nvfp4", 512, "last"), ("int8", 256, "first"), ("bf16", 208, "last")])
def test_fused_amax_feeds_quant(kind, K, where, orc):
    require_gpu()
    M, N = 600, 528
    say(f"fused amax {kind} M={M} N={N} K={K} planted={where}")
    args, _ = _inputs(orc, kind, M, N, K, seed=3 * K + len(where), where=where)
    for epi in (dm.EPI_NVFP4_AMAX, dm.EPI_NVFP4_AMAX | dm.EPI_GELU):
        ws = dm.new_workspace(dm.OP_GEMM_AMAX, "cuda", M, N)
        ws.fill_(0xFF)  # NaN bytes: every slot read must have been written
        y = _run(kind, args, M, N, epi, ws)
        # the stored output equals the epilogue's plain counterpart
        y_plain = _run(kind, args, M, N, epi & dm.EPI_GELU, None)
        assert np.array_equal(y, y_plain)
        tiles = (-(-M // 256)) * (-(-N // 256))
        parts = np.sort(host(ws, np.uint8)[:4 * tiles].view(np.float32))
        assert np.array_equal(parts, _hadamard_tile_max(y, M, N))
        # given-amax quantization == the two-pass quantization of the same y
        yd = dev(y)
        out = []
        for flags, w in ((dm.AMAX_GIVEN, ws), (0, dm.new_workspace(dm.OP_QUANT_NVFP4))):
            codes, scales = empty((M, N // 2), np.uint8), empty((M, N // 16), np.uint8)
            g = empty((1,), np.float32)
            dm.hadamard_quant_nvfp4(yd, codes, scales, g, w, flags)
            torch.cuda.synchronize()
            out.append((host(codes), host(scales), host(g)))
        for a, b in zip(*out):
            assert np.array_equal(a, b)
        assert out[0][2][0] > 0


def test_fused_amax_small_and_single_tile(orc):
    """One partial tile (M, N < 256) and one row: the fold sees one slot."""
    require_gpu()
    for M, N, K in ((1, 16, 256), (37, 48, 208), (256, 256, 512)):
        say(f"fused amax small M={M} N={N} K={K}")
        args, _ = _inputs(orc, "nvfp4", M, N, K, seed=M + N)
        ws = dm.new_workspace(dm.OP_GEMM_AMAX, "cuda", M, N)
        y = _run("nvfp4", args, M, N, dm.EPI_NVFP4_AMAX, ws)
        tiles = (-(-M // 256)) * (-(-N // 256))
        parts = np.sort(host(ws, np.uint8)[:4 * tiles].view(np.float32))
        assert np.array_equal(parts, _hadamard_tile_max(y, M, N))
        out = []
        for flags, w in ((dm.AMAX_GIVEN, ws), (0, dm.new_workspace(dm.OP_QUANT_NVFP4))):
            codes, scales = empty((M, N // 2), np.uint8), empty((M, N // 16), np.uint8)
            g = empty((1,), np.float32)
            dm.hadamard_quant_nvfp4(dev(y), codes, scales, g, w, flags)
            torch.cuda.synchronize()
            out.append((host(codes), host(scales), host(g)))
        for a, b in zip(*out):
            assert np.array_equal(a, b)


def test_fused_epilogue_empty():
    require_gpu()
    ws = dm.new_workspace(dm.OP_GEMM_AMAX, "cuda", 0, 32)
    dm.gemm_bf16_ex(empty((0, 32), np.uint16), empty((32, 32), np.uint16), empty((0, 32), np.uint16),
                    dm.EPI_NVFP4_AMAX | dm.EPI_GELU, ws)
    codes, scales, g = empty((0, 16), np.uint8), empty((0, 2), np.uint8), empty((1,), np.float32)
    g.fill_(7.0)
    dm.hadamard_quant_nvfp4(empty((0, 32), np.uint16), codes, scales, g, ws, dm.AMAX_GIVEN)
    torch.cuda.synchronize()
    assert host(g)[0] == 0.0
