"""GPU parity of the tail split along K: the *_ex GEMMs with a full GEMM
workspace (DMPQ_OP_GEMM) split the tiles beyond the last multiple of 256
along K (by stages of 256 K elements; an NVFP4 K that is a multiple of
128 but not of 256 ends with a half stage) and add the parts in a fixed order in a second kernel.

INT8: int32 parts add exactly, so the outputs are bit-exact against the
oracle and bit-identical to the unsplit call.  NVFP4 and BF16: the same
per-element bound as the unsplit GEMMs (1e-5 * B), and the same bits on a
repeated call (the fixed summation order).  Shapes: a lone partial wave
(every tile split), full waves plus a tail, the CogVideoX-like full shapes
the bench times (row sample that includes every tail tile's rows), a BF16 K
tail inside the last split, and the fused epilogues on split tiles.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, empty, host, require_gpu, say
from test_gpu_fused import _hadamard_tile_max

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _splits(M, N, nk):
    """The split factor the library's plan picks (1: no split)."""
    tiles = (-(-M // 256)) * (-(-N // 256))
    tail = tiles % 256
    if tail == 0:
        return 1
    s = min(256 // tail, nk)
    s = 8 if s >= 8 else 4 if s >= 4 else s    # the fixup exists for 2, 3, 4 and 8 parts
    return s if s >= 2 else 1


def _rows(M):
    return np.unique(np.concatenate([np.arange(0, M, 211), np.arange(max(M - 3, 0), M)]))


def _sel(rows):
    return slice(None) if rows is None else torch.from_numpy(rows).cuda()


def _gemm_ws(M, N):
    return dm.new_workspace(dm.OP_GEMM, "cuda", M, N)


@pytest.mark.parametrize("M,N,K,sample", [(600, 528, 4096, False), (600, 528, 1024, False),
                                          (1792, 1536, 4096, False), (4352, 4096, 4096, True),
                                          (4096, 2048, 4096, False),
                                          (workloads.M_480P, 3072, 12288, True),
                                          (workloads.M_480P, 3072, 3072, True)])
def test_split_int8(orc, M, N, K, sample):
    """INT8 splits from K = 4096 on; below that the same call runs unsplit."""
    require_gpu()
    S = _splits(M, N, K // 128) if K >= 4096 else 1
    if (M, N, K) == (4096, 2048, 4096):
        assert S == 2                  # 128 tiles: the two-way fixup
    say(f"split int8 M={M} N={N} K={K} splits={S}")
    rng = np.random.default_rng(M + N + K)
    qa, sa = orc.quant_int8(workloads.activations(rng, M, K))
    p = orc.prep_weight(workloads.weight(rng, N, K))
    rows = _rows(M) if sample else None
    _, y0 = orc.gemm_int8(qa, sa, p["qw"], p["sw_row"], rows=rows)
    args = (dev(qa), dev(sa), dev(p["qw"]), dev(p["sw_row"]))
    ws = _gemm_ws(M, N)
    for out, dt in ((dm.OUT_F32, np.float32), (dm.OUT_BF16, np.uint16)):
        y = empty((M, N), dt)
        dm.qgemm_int8_ex(*args, y, 0, ws, out)
        yp = empty((M, N), dt)
        dm.qgemm_int8(*args, yp, out)
        torch.cuda.synchronize()
        assert torch.equal(y, yp)
        got = host(y[_sel(rows)], dt)
        want = y0 if out == dm.OUT_F32 else workloads.to_bf16_bits(y0)
        assert np.array_equal(got.view(np.uint32 if dt == np.float32 else np.uint16),
                              want.view(np.uint32 if dt == np.float32 else np.uint16))


def _run_fp4(args, M, N, ws, out=dm.OUT_F32):
    y = empty((M, N), np.float32 if out == dm.OUT_F32 else np.uint16)
    dm.qgemm_nvfp4_ex(*args, y, 0, ws, out)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("M,N,K,sample", [(600, 528, 512, False), (600, 528, 2048, False),
                                          (600, 528, 1920, False), (600, 528, 384, False),
                                          (4352, 4096, 1024, True),
                                          (workloads.M_480P, 3072, 12288, True),
                                          (workloads.M_480P, 12288, 3072, True),
                                          (workloads.M_480P, 3072, 3072, True),
                                          (workloads.M_480P, 1920, 1920, True)])
def test_split_nvfp4(orc, M, N, K, sample):
    # K % 256 == 0 runs 256-element stages; other K % 128 == 0 adds a half stage
    require_gpu()
    S = _splits(M, N, K // 256 + (1 if K % 256 else 0))
    say(f"split nvfp4 M={M} N={N} K={K} splits={S}")
    assert S > 1
    rng = np.random.default_rng(2 * M + N + K)
    ca, sa, ga = orc.quant_nvfp4(workloads.activations(rng, M, K))
    p = orc.prep_weight(workloads.weight(rng, N, K))
    rows = _rows(M) if sample else None
    y0, b0 = orc.gemm_nvfp4(ca, sa, ga, p["cw"], p["sw"], p["gw"], rows=rows)
    args = (dev(ca), dev(sa), dev(np.array([ga], np.float32)), dev(p["cw"]), dev(p["sw"]),
            dev(np.array([p["gw"]], np.float32)))
    ws = _gemm_ws(M, N)
    y = _run_fp4(args, M, N, ws)
    assert torch.equal(y, _run_fp4(args, M, N, ws))          # deterministic
    got = host(y[_sel(rows)]).astype(np.float64)
    err = np.abs(got - y0)
    assert np.all(err <= TOL * b0), float((err / np.maximum(b0, 1e-300)).max())
    yb = workloads.bf16_bits_to_f32(host(_run_fp4(args, M, N, ws, dm.OUT_BF16)[_sel(rows)],
                                         np.uint16)).astype(np.float64)
    assert np.all(np.abs(yb - y0) <= TOL * b0 + 2.0 ** -8 * np.abs(y0))


@pytest.mark.parametrize("M,N,K,sample", [(600, 528, 256, False), (600, 528, 208, False),
                                          (4352, 4096, 208, True), (4352, 4096, 1024, True)])
def test_split_bf16(orc, M, N, K, sample):
    require_gpu()
    S = _splits(M, N, -(-2 * K // 128))
    say(f"split bf16 M={M} N={N} K={K} splits={S}")
    assert S > 1
    rng = np.random.default_rng(3 * M + N + K)
    x = workloads.activations(rng, M, K)
    w = workloads.weight(rng, N, K)
    rows = _rows(M) if sample else None
    y0, b0 = orc.gemm_bf16(x, w, rows=rows)
    ws = _gemm_ws(M, N)
    y = empty((M, N), np.float32)
    dm.gemm_bf16_ex(dev(x), dev(w), y, 0, ws, dm.OUT_F32)
    y2 = empty((M, N), np.float32)
    dm.gemm_bf16_ex(dev(x), dev(w), y2, 0, ws, dm.OUT_F32)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    err = np.abs(host(y[_sel(rows)]).astype(np.float64) - y0)
    assert np.all(err <= TOL * b0), float((err / np.maximum(b0, 1e-300)).max())


@pytest.mark.parametrize("kind,K", [("int8", 4096), ("nvfp4", 2048), ("nvfp4", 1920), ("bf16", 208)])
def test_split_with_fused_epilogue(orc, kind, K):
    """GELU + amax on split tiles: the output equals the unsplit fused call's
    (INT8) or its GELU of the split pre-activation, and the per-tile maxima
    are the tiles' own, so the given-amax quantization matches the two-pass
    one bit for bit."""
    require_gpu()
    M, N = 600, 528
    say(f"split + fused epilogue {kind} M={M} N={N} K={K}")
    rng = np.random.default_rng(K + 5)
    x = workloads.activations(rng, M, K)
    w = workloads.weight(rng, N, K)
    ws = _gemm_ws(M, N)
    epi = dm.EPI_GELU | dm.EPI_NVFP4_AMAX

    def run(e, wsp):
        y = empty((M, N), np.uint16)
        if kind == "int8":
            qa, sa = orc.quant_int8(x)
            p = orc.prep_weight(w)
            dm.qgemm_int8_ex(dev(qa), dev(sa), dev(p["qw"]), dev(p["sw_row"]), y, e, wsp)
        elif kind == "nvfp4":
            ca, sa, ga = orc.quant_nvfp4(x)
            p = orc.prep_weight(w)
            dm.qgemm_nvfp4_ex(dev(ca), dev(sa), dev(np.array([ga], np.float32)), dev(p["cw"]),
                              dev(p["sw"]), dev(np.array([p["gw"]], np.float32)), y, e, wsp)
        else:
            dm.gemm_bf16_ex(dev(x), dev(w), y, e, wsp)
        torch.cuda.synchronize()
        return y

    ws.fill_(0xFF)
    y = run(epi, ws)
    tiles = (-(-M // 256)) * (-(-N // 256))
    parts = np.sort(host(ws[:4 * tiles], np.uint8).view(np.float32))
    yh = host(y, np.uint16)
    assert np.array_equal(parts, _hadamard_tile_max(yh, M, N))
    assert torch.equal(y, run(dm.EPI_GELU, ws))               # the same split, GELU only
    if kind == "int8":
        small = dm.new_workspace(dm.OP_GEMM_AMAX, "cuda", M, N)   # too small to split
        assert torch.equal(y, run(epi, small))
    out = []
    for flags, wq in ((dm.AMAX_GIVEN, None), (0, dm.new_workspace(dm.OP_QUANT_NVFP4))):
        if wq is None:
            run(epi, ws)                                      # refresh the maxima
            wq = ws
        codes, scales = empty((M, N // 2), np.uint8), empty((M, N // 16), np.uint8)
        g = empty((1,), np.float32)
        dm.hadamard_quant_nvfp4(y, codes, scales, g, wq, flags)
        torch.cuda.synchronize()
        out.append((host(codes), host(scales), host(g)))
    for a, b in zip(*out):
        assert np.array_equal(a, b)
