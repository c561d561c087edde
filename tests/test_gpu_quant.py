"""GPU parity: Hadamard + INT8 / NVFP4 activation quantization and weight prep
against the oracle, bit for bit (codes, scales, tensor scale)."""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, empty, host, require_gpu, say

pytestmark = pytest.mark.gpu

SHAPES = [(1, 16), (37, 16), (37, 48), (5, 256), (256, 256), (37, 1920), (19, 3072),
          (11, 7680), (9, 12288), (3, 16400), (2, 32768)]


def _gpu_int8(x, flags=0):
    M, K = x.shape
    q, s = empty((M, K), np.int8), empty((M,), np.float32)
    dm.hadamard_quant_int8(dev(x).view(M, K), q, s, flags=flags)
    torch.cuda.synchronize()
    return host(q), host(s)


def _gpu_nvfp4(x, flags=0):
    M, K = x.shape
    c, s = empty((M, K // 2), np.uint8), empty((M, K // 16), np.uint8)
    g = torch.full((1,), -1.0, device="cuda")
    ws = dm.new_workspace(dm.OP_QUANT_NVFP4)
    dm.hadamard_quant_nvfp4(dev(x).view(M, K), c, s, g, ws, flags=flags)
    torch.cuda.synchronize()
    return host(c), host(s), float(host(g)[0])


def _check_int8(orc, x, flags=0):
    q0, s0 = orc.quant_int8(x, flags)
    q1, s1 = _gpu_int8(x, flags)
    assert np.array_equal(s1.view(np.uint32), s0.view(np.uint32))
    assert np.array_equal(q1, q0)


def _check_nvfp4(orc, x, flags=0):
    c0, s0, g0 = orc.quant_nvfp4(x, flags)
    c1, s1, g1 = _gpu_nvfp4(x, flags)
    assert np.float32(g1).view(np.uint32) == np.float32(g0).view(np.uint32)
    assert np.array_equal(s1, s0)
    assert np.array_equal(c1, c0)


@pytest.mark.parametrize("M,K", SHAPES)
def test_int8_quant_parity(orc, M, K):
    require_gpu()
    say(f"hadamard_quant_int8 M={M} K={K}")
    x = workloads.activations(np.random.default_rng(M * 7 + K), M, K)
    _check_int8(orc, x)
    _check_int8(orc, x, dm.NO_HADAMARD)


@pytest.mark.parametrize("M,K", SHAPES)
def test_nvfp4_quant_parity(orc, M, K):
    require_gpu()
    say(f"hadamard_quant_nvfp4 M={M} K={K}")
    x = workloads.activations(np.random.default_rng(M * 11 + K), M, K)
    _check_nvfp4(orc, x)
    _check_nvfp4(orc, x, dm.NO_HADAMARD)


def test_quant_edge_cases(orc):
    require_gpu()
    say("quant edge cases: zero rows, zero tensor, tiny and huge values, M=0")
    rng = np.random.default_rng(60)
    x = workloads.activations(rng, 40, 256)
    x[3] = 0
    x[17, 5:40] = 0
    _check_int8(orc, x)
    _check_nvfp4(orc, x)
    z = np.zeros((9, 64), np.uint16)
    _check_int8(orc, z)
    _check_nvfp4(orc, z)
    # wide dynamic range: tiny blocks next to huge ones (scale underflow to 0)
    f = rng.standard_normal((16, 128)).astype(np.float32)
    f[:, :16] *= np.float32(1e30)
    f[:, 16:32] *= np.float32(1e-30)
    xr = workloads.to_bf16_bits(f)
    _check_int8(orc, xr)
    _check_nvfp4(orc, xr)
    # empty input is a no-op
    q, s = empty((0, 64), np.int8), empty((0,), np.float32)
    dm.hadamard_quant_int8(empty((0, 64), np.uint16), q, s)
    c, sc = empty((0, 32), np.uint8), empty((0, 4), np.uint8)
    g = torch.zeros(1, device="cuda")
    dm.hadamard_quant_nvfp4(empty((0, 64), np.uint16), c, sc, g, dm.new_workspace(1))
    torch.cuda.synchronize()
    assert float(g[0]) == 0.0


def test_nvfp4_grid_roundtrip_gpu(orc):
    # tensor on the NVFP4 grid with g = 1 (see the oracle pins): GPU recovers it
    require_gpu()
    say("nvfp4 grid round trip")
    from test_oracle_quant import _nvfp4_grid_tensor
    xb, codes, e = _nvfp4_grid_tensor(orc, np.random.default_rng(61), 12, 96)
    c, s, g = _gpu_nvfp4(xb, dm.NO_HADAMARD)
    assert g == 1.0 and np.array_equal(s, e) and np.array_equal(c, codes)


@pytest.mark.parametrize("K", [1920, 3072, 7680, 12288])
def test_quant_full_token_count(orc, K):
    # every row of a CogVideoX-like 17776-token activation
    require_gpu()
    M = workloads.M_480P
    say(f"full-size quant M={M} K={K}")
    x = workloads.activations(np.random.default_rng(K), M, K)
    _check_int8(orc, x)
    _check_nvfp4(orc, x)


def test_quant_1080p_tokens(orc):
    require_gpu()
    M, K = workloads.M_1080P, 3072
    say(f"full-size quant M={M} K={K}")
    x = workloads.activations(np.random.default_rng(1080), M, K)
    _check_int8(orc, x)
    _check_nvfp4(orc, x)


@pytest.mark.parametrize("mode", [dm.W8_FROM_NVFP4, dm.W8_DIRECT])
@pytest.mark.parametrize("N,K", [(256, 256), (5760, 1920), (48, 12288), (33, 80)])
def test_prep_weight_parity(orc, mode, N, K):
    require_gpu()
    say(f"prep_weight mode={mode} N={N} K={K}")
    w = workloads.weight(np.random.default_rng(N + K), N, K)
    ref = orc.prep_weight(w, mode)
    cw, sw = empty((N, K // 2), np.uint8), empty((N, K // 16), np.uint8)
    gw = torch.zeros(1, device="cuda")
    qw, swr = empty((N, K), np.int8), empty((N,), np.float32)
    dm.prep_weight(dev(w).view(N, K), cw, sw, gw, qw, swr, dm.new_workspace(dm.OP_PREP_WEIGHT),
                   int8_mode=mode)
    torch.cuda.synchronize()
    assert np.float32(host(gw)[0]).view(np.uint32) == np.float32(ref["gw"]).view(np.uint32)
    assert np.array_equal(host(cw), ref["cw"]) and np.array_equal(host(sw), ref["sw"])
    assert np.array_equal(host(swr).view(np.uint32), ref["sw_row"].view(np.uint32))
    assert np.array_equal(host(qw), ref["qw"])


@pytest.mark.parametrize("N,K", [(1, 16), (33, 96), (5760, 1920), (70, 12288), (9216, 3072)])
def test_weight_int8_from_nvfp4_parity(orc, N, K):
    # the conversion an INT8-routed linear runs on its NVFP4 weight: bit-exact
    # against the oracle, and identical to what dmpq_prep_weight stores
    require_gpu()
    say(f"weight_int8_from_nvfp4 N={N} K={K}")
    w = workloads.weight(np.random.default_rng(3 * N + K), N, K)
    ref = orc.prep_weight(w)
    qw, swr = empty((N, K), np.int8), empty((N,), np.float32)
    dm.weight_int8_from_nvfp4(dev(ref["cw"]), dev(ref["sw"]), dev(np.array([ref["gw"]], np.float32)),
                              qw, swr)
    torch.cuda.synchronize()
    assert np.array_equal(host(qw), ref["qw"])
    assert np.array_equal(host(swr).view(np.uint32), ref["sw_row"].view(np.uint32))


def test_weight_int8_from_nvfp4_random_codes(orc):
    # arbitrary codes, every finite E4M3 scale, tensor scales far from 1, an
    # all-zero row, and the non-finite tensor scales (+inf: rows of +-inf and
    # NaN values; NaN: all-NaN rows)
    require_gpu()
    say("weight_int8_from_nvfp4 random codes")
    rng = np.random.default_rng(63)
    N, K = 130, 2080
    cw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sw = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    cw[5] = 0
    gvals = np.array([3.0517578e-05, 0.75, 1.7e3, 2.0 ** 101, 3e38, np.inf, np.nan], np.float32)
    # and NaNs whose low payload byte is not zero (quiet and signalling)
    gvals = np.concatenate([gvals, np.array([0x7FC000A5, 0x7F800001], np.uint32).view(np.float32)])
    for g in gvals:
        q_ref, s_ref = orc.w8_from_nvfp4(cw, sw, g)
        qw, swr = empty((N, K), np.int8), empty((N,), np.float32)
        dm.weight_int8_from_nvfp4(dev(cw), dev(sw), dev(np.array([g], np.float32)), qw, swr)
        torch.cuda.synchronize()
        assert np.array_equal(host(qw), q_ref)
        assert np.array_equal(host(swr).view(np.uint32), s_ref.view(np.uint32))
        assert np.all(host(qw)[5] == 0) and host(swr)[5] == 0


def _int8_w8_call(x, cw, sw, g, flags=0):
    M, K = x.shape
    N = cw.shape[0]
    q, s = empty((M, K), np.int8), empty((M,), np.float32)
    qw, swr = empty((N, K), np.int8), empty((N,), np.float32)
    dm.hadamard_quant_int8_w8(dev(x).view(M, K), q, s, dev(cw).view(N, K // 2), dev(sw).view(N, K // 16),
                              dev(np.array([g], np.float32)), qw, swr, flags=flags)
    torch.cuda.synchronize()
    return host(q), host(s), host(qw), host(swr)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (37, 33, 96), (300, 200, 3072), (19, 70, 12288),
                                   (0, 33, 96), (37, 0, 96), (17776, 9216, 3072), (17776, 3072, 12288)])
def test_int8_w8_one_launch_parity(orc, M, N, K):
    # the INT8 route's activation quantization and weight conversion in one
    # launch: each output bit-exact against the oracle (the 5B-like qkv and
    # ffn_down shapes included)
    require_gpu()
    say(f"hadamard_quant_int8_w8 M={M} N={N} K={K}")
    rng = np.random.default_rng(5 * M + 3 * N + K)
    x = workloads.activations(rng, M, K)
    ref = orc.prep_weight(workloads.weight(rng, N, K))
    flag_set = (0, dm.NO_HADAMARD) if M * K <= 1 << 20 else (0,)
    for flags in flag_set:
        q, s, qw, swr = _int8_w8_call(x, ref["cw"], ref["sw"], ref["gw"], flags)
        q0, s0 = orc.quant_int8(x, flags)
        assert np.array_equal(s.view(np.uint32), s0.view(np.uint32))
        assert np.array_equal(q, q0)
        assert np.array_equal(qw, ref["qw"])
        assert np.array_equal(swr.view(np.uint32), ref["sw_row"].view(np.uint32))


def test_int8_w8_one_launch_weight_rules(orc):
    # arbitrary codes and scales, an all-zero weight row, and tensor scales
    # that are tiny, huge, infinite and NaN: the weight half follows the
    # conversion's rules exactly, beside a ragged activation half
    require_gpu()
    say("hadamard_quant_int8_w8 weight rules")
    rng = np.random.default_rng(64)
    M, N, K = 45, 130, 2080
    x = workloads.activations(rng, M, K)
    cw = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sw = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    cw[5] = 0
    q0, s0 = orc.quant_int8(x, 0)
    for g in np.array([3.0517578e-05, 1.7e3, 2.0 ** 101, np.inf, np.nan], np.float32):
        q, s, qw, swr = _int8_w8_call(x, cw, sw, g)
        qw0, swr0 = orc.w8_from_nvfp4(cw, sw, g)
        assert np.array_equal(qw, qw0)
        assert np.array_equal(swr.view(np.uint32), swr0.view(np.uint32))
        assert np.array_equal(q, q0) and np.array_equal(s.view(np.uint32), s0.view(np.uint32))


def test_quant_subnormal_inputs(orc):
    # bf16 subnormals (below 2^-126) must be kept, not flushed, through the
    # Hadamard and both quantizers
    require_gpu()
    say("quant with subnormal inputs")
    rng = np.random.default_rng(62)
    f = rng.standard_normal((8, 64)).astype(np.float32) * np.float32(1e-39)
    f[:, :16] = rng.standard_normal((8, 16)).astype(np.float32)
    x = workloads.to_bf16_bits(f)
    _check_int8(orc, x)
    _check_nvfp4(orc, x)
    xs = workloads.to_bf16_bits(rng.standard_normal((8, 64)).astype(np.float32) * np.float32(1e-39))
    _check_int8(orc, xs)
    _check_nvfp4(orc, xs)


def test_quant_non_finite_inputs(orc):
    """The non-finite rule (a NaN codes 0 and never enters an amax; an infinity
    makes its row's or tensor's amax infinite, so its scale is +inf and its
    codes 0), on rows with quiet and signalling NaNs of both signs, single
    infinities (every rotated output infinite) and pairs of opposite
    infinities in one block (NaN and infinite outputs), with and without the
    Hadamard."""
    require_gpu()
    say("quant with NaN and infinite inputs")
    rng = np.random.default_rng(64)
    M, K = 24, 96
    x = workloads.activations(rng, M, K)
    nans = (0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FFF)
    for i, r in enumerate(range(0, 10, 2)):
        x[r, 7 * i + 3] = nans[i]
    x[11, 40] = 0x7F80
    x[13, 50] = 0xFF80
    x[15, 16], x[15, 17] = 0x7F80, 0xFF80
    x[17, 32:48] = 0x7FC0
    for flags in (0, dm.NO_HADAMARD):
        _check_int8(orc, x, flags)
    # NVFP4's amax is tensor-wide: NaNs alone (finite amax), then an infinity
    xn = x.copy()
    xn[11, 40] = xn[13, 50] = xn[15, 16] = xn[15, 17] = 0x3F80
    for flags in (0, dm.NO_HADAMARD):
        _check_nvfp4(orc, xn, flags)
        _check_nvfp4(orc, x, flags)
    c, s, g = _gpu_nvfp4(x)
    assert g == np.inf and not c.any() and not s.any()
