"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/dmpq.h declares, its host-side functions (router, TDC decide/commit)
agree with the oracle, and argument errors are reported before any launch.
"""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import dynamic_mixed_precision_amd as dm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "dmpq.h")).read()
    return sorted(set(re.findall(r"\b(dmpq_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = dm.lib()
    names = _declared()
    assert len(names) >= 14
    for name in names:
        assert hasattr(L, name), name
    assert sorted(dm.EXPORTS) == names


def test_version_and_workspace():
    assert "gfx950" in dm.version()
    for op in (dm.OP_GAMMA, dm.OP_QUANT_NVFP4, dm.OP_TDC, dm.OP_PREP_WEIGHT):
        assert dm.workspace_bytes(op, 17776, 3072) >= 2048 * 4 * 8
    assert dm.workspace_bytes(99) == 0


def test_router_matches_oracle(orc):
    rng = np.random.default_rng(50)
    for _ in range(300):
        n = int(rng.integers(1, 8))
        alpha = rng.uniform(-2, 3, n)
        beta = rng.uniform(-0.5, 0.5, n)
        tau = float(rng.uniform(-0.2, 0.8))
        sums = rng.uniform(0, 10, 2)
        if rng.random() < 0.1:
            sums[1] = 0.0
        g0, e0, r0 = orc.route(sums, alpha, beta, tau)
        g1, e1, r1 = dm.gate_and_route(sums, alpha, beta, tau)
        assert (g0 == g1) or (math.isinf(g0) and math.isinf(g1))
        assert np.array_equal(np.nan_to_num(e0), np.nan_to_num(e1))
        assert np.array_equal(r0, r1)
    g, e, r = dm.gate_and_route(None, [1.0, 2.0], [0.0, 0.0], 0.1)
    assert math.isnan(g) and np.all(r == dm.ROUTE_INT8)
    # exact tie -> NVFP4
    _, _, r = dm.gate_and_route([1.0, 4.0], [1.0], [0.0], 0.25)
    assert r[0] == dm.ROUTE_NVFP4


def test_tdc_bookkeeping_matches_oracle(orc):
    rng = np.random.default_rng(51)
    eps, dacc = 0.3, 0.7
    so, sl = orc.tdc_new(), dm.tdc_init()
    for t in range(200):
        skip_o = orc.tdc_decide(so, eps, dacc)
        skip_l = dm.tdc_decide(sl, eps, dacc)
        assert skip_o == skip_l, t
        if skip_o:
            orc.tdc_commit_skip(so)
            dm.tdc_commit(sl, dm.TDC_SKIP)
        else:
            sums = rng.uniform(0, 1, 4)
            sums[2] *= rng.choice([0.1, 1.0])
            orc.tdc_commit_refresh(so, sums)
            dm.tdc_commit(sl, dm.TDC_REFRESH, sums)
        for f in ("n_refresh", "d", "acc", "delta_valid", "gamma_valid"):
            assert getattr(so, f) == getattr(sl, f), (t, f)


class _Fake:
    """Stands in for a device tensor in calls that must fail validation."""

    def __init__(self, shape, addr=0x10000, numel=None):
        self.shape = shape
        self._addr = addr
        self._n = numel if numel is not None else int(np.prod(shape))
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self._addr

    def numel(self):
        return self._n


def _expect(status, fn, *args, **kw):
    with pytest.raises(dm.DmpqError) as ei:
        fn(*args, **kw)
    assert ei.value.status == status
    assert dm.last_error()


def _library_checks_only(monkeypatch):
    """The fakes carry shapes but no element sizes: skip the binding's own size
    checks so that each call reaches the library's validation."""
    monkeypatch.setattr(dm, "_stream", lambda s=None: 0)
    monkeypatch.setattr(dm, "_need", lambda *a, **k: None)


def test_validation_before_launch(monkeypatch):
    _library_checks_only(monkeypatch)
    x = _Fake((4, 24))
    _expect(2, dm.hadamard_quant_int8, x, _Fake((4, 24)), _Fake((4,)))           # K % 16
    _expect(3, dm.hadamard_quant_int8, _Fake((4, 32), addr=0x10008), _Fake((4, 32)), _Fake((4,)))
    _expect(1, dm.hadamard_quant_int8, _Fake((4, 32)), _Fake((4, 32)), _Fake((4,)), flags=6)
    _expect(4, dm.hadamard_quant_int8, _Fake((4, 65536)), _Fake((4, 65536)), _Fake((4,)))
    ws_small = _Fake((16,), numel=16)
    _expect(6, dm.hadamard_quant_nvfp4, _Fake((4, 32)), _Fake((4, 16)), _Fake((4, 2)), _Fake((1,)),
            ws_small)
    _expect(2, dm.qgemm_int8, _Fake((4, 40)), _Fake((4,)), _Fake((8, 40)), _Fake((8,)), _Fake((4, 8)))
    _expect(1, dm.qgemm_int8, _Fake((4, 64)), _Fake((4,)), _Fake((8, 64)), _Fake((8,)),
            _Fake((4, 8)), out_dtype=7)
    _expect(1, dm.qgemm_nvfp4, _Fake((4, 32)), _Fake((4, 4)), _Fake((1,)), _Fake((8, 32)),
            _Fake((8, 4)), _Fake((1,)), _Fake((4, 8)), variant=5)
    _expect(1, dm.tdc_step, 9, _Fake((64,)), _Fake((64,)), _Fake((64,)), True)
    _expect(1, dm.tdc_step, dm.TDC_SKIP, _Fake((64,)), _Fake((64,)), _Fake((64,)), False)
    _expect(6, dm.tdc_step, dm.TDC_REFRESH, _Fake((64,)), _Fake((64,)), _Fake((64,)), True,
            sums=_Fake((4,)), ws=None)
    _expect(1, dm.prep_weight, _Fake((8, 32)), _Fake((8, 16)), _Fake((8, 2)), _Fake((1,)),
            _Fake((8, 32)), _Fake((8,)), _Fake((65792,)), int8_mode=3)
    # cw [N x K/2]: K = 2 * 12 = 24 is not a multiple of 16; K = 2 * 32768 is too large
    _expect(2, dm.weight_int8_from_nvfp4, _Fake((8, 12)), _Fake((8, 1)), _Fake((1,)),
            _Fake((8, 24)), _Fake((8,)))
    _expect(4, dm.weight_int8_from_nvfp4, _Fake((8, 32768)), _Fake((8, 4096)), _Fake((1,)),
            _Fake((8, 65536)), _Fake((8,)))
    _expect(3, dm.weight_int8_from_nvfp4, _Fake((8, 16)), _Fake((8, 2)), _Fake((1,), addr=0x10004),
            _Fake((8, 32)), _Fake((8,)))
    # the one-launch INT8 route: activation and weight rules together
    xw = (_Fake((4, 32)), _Fake((4, 32)), _Fake((4,)))
    ww = (_Fake((8, 16)), _Fake((8, 2)), _Fake((1,)), _Fake((8, 32)), _Fake((8,)))
    _expect(2, dm.hadamard_quant_int8_w8, _Fake((4, 24)), _Fake((4, 24)), _Fake((4,)), _Fake((8, 12)),
            _Fake((8, 1)), _Fake((1,)), _Fake((8, 24)), _Fake((8,)))
    _expect(1, dm.hadamard_quant_int8_w8, *xw, *ww, flags=6)
    _expect(3, dm.hadamard_quant_int8_w8, *xw, _Fake((8, 16)), _Fake((8, 2)), _Fake((1,), addr=0x10004),
            _Fake((8, 32)), _Fake((8,)))
    _expect(3, dm.hadamard_quant_int8_w8, _Fake((4, 32), addr=0x10008), _Fake((4, 32)), _Fake((4,)), *ww)
    _expect(4, dm.hadamard_quant_int8_w8, _Fake((4, 65536)), _Fake((4, 65536)), _Fake((4,)),
            _Fake((8, 32768)), _Fake((8, 4096)), _Fake((1,)), _Fake((8, 65536)), _Fake((8,)))


def test_fused_epilogue_validation(monkeypatch):
    """Producer-epilogue GEMMs and the quantizer's given-amax flag reject
    bad combinations before any launch."""
    _library_checks_only(monkeypatch)
    M, N, K = 300, 48, 64
    qa, sa, qw, sw = _Fake((M, K)), _Fake((M,)), _Fake((N, K)), _Fake((N,))
    y = _Fake((M, N))
    need = dm.workspace_bytes(dm.OP_GEMM_AMAX, M, N)
    assert need >= 4 * 2 * 1 and need >= dm.workspace_bytes(dm.OP_QUANT_NVFP4)
    # 2^20 x 2^16 outputs = 16384 tiles: the size grows past the fixed workspace
    assert dm.workspace_bytes(dm.OP_GEMM_AMAX, 1 << 20, 1 << 16) == 4 * 4096 * 256
    assert dm.workspace_bytes(dm.OP_GEMM_AMAX, -1, 16) == 0
    # full GEMM workspace: the tile maxima rounded up to 256 bytes, then 64 MiB
    assert dm.workspace_bytes(dm.OP_GEMM, M, N) == 256 + (64 << 20)
    assert dm.workspace_bytes(dm.OP_GEMM, 17776, 3072) == 3584 + (64 << 20)
    _expect(1, dm.qgemm_int8_ex, qa, sa, qw, sw, y, 0, out_dtype=5)
    _expect(1, dm.qgemm_nvfp4_ex, _Fake((M, K // 2)), _Fake((M, K // 16)), _Fake((1,)),
            _Fake((N, K // 2)), _Fake((N, K // 16)), _Fake((1,)), y, 0, out_dtype=dm.OUT_I32)
    _expect(3, dm.gemm_bf16_ex, _Fake((M, K)), _Fake((N, K)), y, 0,
            ws=_Fake((need,), numel=need, addr=0x10004))
    _expect(1, dm.qgemm_int8_ex, qa, sa, qw, sw, y, 4)                          # unknown bit
    _expect(4, dm.qgemm_int8_ex, qa, sa, qw, sw, y, dm.EPI_GELU, out_dtype=dm.OUT_F32)
    _expect(2, dm.qgemm_int8_ex, qa, sa, _Fake((40, K)), _Fake((40,)), _Fake((M, 40)),
            dm.EPI_NVFP4_AMAX, ws=_Fake((need,), numel=need))                   # N % 16
    _expect(6, dm.qgemm_int8_ex, qa, sa, qw, sw, y, dm.EPI_NVFP4_AMAX)          # no workspace
    _expect(6, dm.qgemm_int8_ex, qa, sa, qw, sw, y, dm.EPI_NVFP4_AMAX, ws=_Fake((4,), numel=4))
    _expect(3, dm.gemm_bf16_ex, _Fake((M, K)), _Fake((N, K)), y, dm.EPI_NVFP4_AMAX,
            ws=_Fake((need,), numel=need, addr=0x10008))
    _expect(4, dm.qgemm_nvfp4_ex, _Fake((M, K // 2)), _Fake((M, K // 16)), _Fake((1,)),
            _Fake((N, K // 2)), _Fake((N, K // 16)), _Fake((1,)), y, dm.EPI_GELU,
            out_dtype=dm.OUT_F32)
    x = _Fake((M, N))
    ws = _Fake((need,), numel=need)
    _expect(1, dm.hadamard_quant_nvfp4, x, _Fake((M, N // 2)), _Fake((M, N // 16)), _Fake((1,)),
            ws, flags=dm.AMAX_GIVEN | dm.NO_HADAMARD)
    _expect(1, dm.hadamard_quant_nvfp4, x, _Fake((M, N // 2)), _Fake((M, N // 16)), _Fake((1,)),
            ws, flags=4)
    big = 1 << 20
    small = dm.workspace_bytes(dm.OP_QUANT_NVFP4)
    _expect(6, dm.hadamard_quant_nvfp4, _Fake((big, 1 << 16)), _Fake((big, 1 << 15)),
            _Fake((big, 1 << 12)), _Fake((1,)), _Fake((small,), numel=small), flags=dm.AMAX_GIVEN)


def test_noalloc_and_w4_gemm_validation(monkeypatch):
    """The no-workspace quantizer and the INT8 GEMM that converts an NVFP4
    weight reject bad arguments before any launch (and their bindings reach
    the library's error path)."""
    _library_checks_only(monkeypatch)
    _expect(2, dm.hadamard_quant_nvfp4_noalloc, _Fake((4, 24)), _Fake((4, 12)), _Fake((4, 1)), _Fake((1,)))
    _expect(4, dm.hadamard_quant_nvfp4_noalloc, _Fake((4, 32)), _Fake((4, 16)), _Fake((4, 2)), _Fake((1,)),
            flags=dm.AMAX_GIVEN)
    M, N, K = 4, 8, 256
    qa, sa, cw, sw, gw, y = (_Fake((M, K)), _Fake((M,)), _Fake((N, K // 2)), _Fake((N, K // 16)), _Fake((1,)),
                             _Fake((M, N)))
    need = dm.workspace_bytes(dm.OP_GEMM_W4, M, N)
    assert need >= 8 * N
    ws = _Fake((need,))
    # K = 192 is not a multiple of 128
    _expect(4, dm.qgemm_int8_from_nvfp4, _Fake((M, 192)), sa, _Fake((N, 96)), _Fake((N, 12)), gw, y, ws)
    _expect(6, dm.qgemm_int8_from_nvfp4, qa, sa, cw, sw, gw, y, None)
    _expect(6, dm.qgemm_int8_from_nvfp4, qa, sa, cw, sw, gw, y, _Fake((need - 1,)))
    _expect(3, dm.qgemm_int8_from_nvfp4, qa, sa, cw, sw, gw, y, _Fake((need,), addr=0x10008))
    _expect(1, dm.qgemm_int8_from_nvfp4, qa, sa, cw, sw, gw, y, ws, epilogue=4)
    _expect(4, dm.qgemm_int8_from_nvfp4, qa, sa, cw, sw, gw, y, ws, epilogue=dm.EPI_GELU, out_dtype=dm.OUT_F32)


def test_gemm_k_limit(monkeypatch):
    """Every GEMM entry point rejects K above 2^22 before any launch (the DMA
    kernels address 256 operand rows by 32-bit offsets)."""
    _library_checks_only(monkeypatch)
    M, N, K = 2, 4, (1 << 22) + 128
    y = _Fake((M, N))
    _expect(4, dm.qgemm_int8, _Fake((M, K)), _Fake((M,)), _Fake((N, K)), _Fake((N,)), y)
    _expect(4, dm.qgemm_nvfp4, _Fake((M, K // 2)), _Fake((M, K // 16)), _Fake((1,)), _Fake((N, K // 2)),
            _Fake((N, K // 16)), _Fake((1,)), y)
    _expect(4, dm.gemm_bf16, _Fake((M, K)), _Fake((N, K)), y)
    ws = _Fake((dm.workspace_bytes(dm.OP_GEMM_W4, M, N),))
    _expect(4, dm.qgemm_int8_from_nvfp4, _Fake((M, K)), _Fake((M,)), _Fake((N, K // 2)), _Fake((N, K // 16)),
            _Fake((1,)), y, ws)


def test_selftest_validation(monkeypatch):
    _library_checks_only(monkeypatch)
    _expect(1, dm.selftest_codec, 2, 0, 16, _Fake((384,)))
    _expect(1, dm.selftest_codec, dm.CODEC_E4M3, 16, 0, _Fake((384,)))
    _expect(1, dm.selftest_codec, dm.CODEC_E2M1, 0, 0x7F800001, _Fake((48,)))


def test_null_pointer_rejected():
    L = dm.lib()
    st = L.dmpq_hadamard_quant_int8(None, None, 4, 32, 0, None, None)
    assert st == 1 and "NULL" in dm.last_error()
    assert L.dmpq_tdc_decide(None, None, None) == 1


def test_binding_checks_buffer_sizes(monkeypatch):
    """The library takes bare pointers, so the binding checks that every tensor
    holds what the call will read or write.  CPU tensors: a call whose sizes
    pass reaches the device-pointer check instead."""
    import torch
    monkeypatch.setattr(dm, "_stream", lambda s=None: 0)
    M, N, K = 8, 32, 64
    i8 = lambda *s: torch.zeros(s, dtype=torch.int8)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)
    bf = lambda *s: torch.zeros(s, dtype=torch.int16)
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)

    def raises(match, fn, *args, **kw):
        with pytest.raises(ValueError, match=match):
            fn(*args, **kw)

    qa, sa, qw, sw = i8(M, K), f32(M), i8(N, K), f32(N)
    raises("GPU tensors", dm.qgemm_int8, qa, sa, qw, sw, f32(M, N))
    raises("y holds", dm.qgemm_int8, qa, sa, qw, sw, f32(M, N - 1))
    raises("y has 4-byte", dm.qgemm_int8, qa, sa, qw, sw, f32(M, N), out_dtype=dm.OUT_BF16)
    raises("qw has shape", dm.qgemm_int8, qa, sa, i8(N, K - 16), sw, f32(M, N))
    raises("sa holds", dm.qgemm_int8_ex, qa, f32(M - 1), qw, sw, bf(M, N))
    ca, sca, g = u8(M, K // 2), u8(M, K // 16), f32(1)
    cw, scw = u8(N, K // 2), u8(N, K // 16)
    raises("GPU tensors", dm.qgemm_nvfp4, ca, sca, g, cw, scw, g, f32(M, N))
    raises("weight scales holds", dm.qgemm_nvfp4, ca, sca, g, cw, u8(N, 1), g, f32(M, N))
    raises("cw has shape", dm.qgemm_nvfp4_ex, ca, sca, g, u8(N, K), scw, g, bf(M, N))
    raises("tensor scale", dm.qgemm_nvfp4, ca, sca, torch.zeros(0), cw, scw, g, f32(M, N))
    raises("w has shape", dm.gemm_bf16, bf(M, K), bf(N, K + 16), f32(M, N))
    raises("x has 1-byte", dm.hadamard_quant_int8, i8(M, K), i8(M, K), f32(M))
    raises("q holds", dm.hadamard_quant_int8, bf(M, K), i8(M, K - 1), f32(M))
    raises("output codes holds", dm.hadamard_quant_nvfp4, bf(M, K), u8(M, K // 4), sca, g, u8(16))
    raises("sums holds", dm.gamma_sums, bf(64), bf(64), torch.zeros(1, dtype=torch.float64), u8(16))
    raises("delta holds", dm.tdc_step, dm.TDC_SKIP, bf(64), bf(64), bf(63), True)
    raises("sums is missing", dm.tdc_step, dm.TDC_REFRESH, bf(64), bf(64), bf(64), False)
    raises("qw holds", dm.weight_int8_from_nvfp4, cw, scw, g, i8(N, K - 1), f32(N))
    raises("qw holds", dm.hadamard_quant_int8_w8, bf(M, K), i8(M, K), f32(M), cw, scw, g, i8(N, K - 1), f32(N))
    raises("s_row holds", dm.hadamard_quant_int8_w8, bf(M, K), i8(M, K), f32(M - 1), cw, scw, g, i8(N, K),
           f32(N))
    raises("cw has shape", dm.hadamard_quant_int8_w8, bf(M, K), i8(M, K), f32(M), u8(N, K), scw, g, i8(N, K),
           f32(N))
    raises("sw_row holds", dm.prep_weight, bf(N, K), cw, scw, g, i8(N, K), f32(N - 1), u8(16))
    raises("count holds", dm.outlier_count, bf(M, K), 4.0, torch.zeros(0, dtype=torch.float64), u8(16))
    raises("stats holds", dm.selftest_codec, dm.CODEC_E4M3, 0, 16, torch.zeros(3 * 128 - 1, dtype=torch.int32))
    raises("stats holds", dm.selftest_codec, dm.CODEC_E2M1, 0, 16, torch.zeros(3 * 16 - 1, dtype=torch.int32))
    raises("stats has 1-byte", dm.selftest_codec, dm.CODEC_E2M1, 0, 16, u8(3 * 16 * 4))
