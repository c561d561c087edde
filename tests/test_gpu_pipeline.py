"""GPU parity of the routed hot path on the CogVideoX-like configurations.

Tiny (256 tokens x 256): Gamma, route, both linears on every row, TDC.

5B-like (17776 tokens, hidden 3072): four synthetic blocks with Gamma about
0.05, 0.40, 0.05, 0.40 route (alpha = 1, beta = 0, tau = 0.2) to NVFP4, INT8,
NVFP4, INT8; the Gamma sums, routes, activation quantization (every row) and
the GEMM (row sample) of each block's linears match the oracle.
2B-like (17776 tokens, hidden 1920): every linear (QKV 5760 x 1920, out
1920 x 1920, FFN up 7680 x 1920, FFN down 1920 x 7680) on both routes, with
the plain entry points and as the benchmark launches them.
1080p-like (106306 tokens): the FFN-up (12288 x 3072) and FFN-down
(3072 x 12288) linears on both routes.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads as wl
from gpu_util import dev, empty, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _rows(M, step):
    return np.unique(np.concatenate([np.arange(0, M, step), np.arange(M - 3, M)]))


def _linear_parity(orc, rng, M, N, K, route, rows):
    x = wl.activations(rng, M, K)
    w = wl.weight(rng, N, K)
    p = orc.prep_weight(w)
    ws = dm.new_workspace(dm.OP_QUANT_NVFP4)
    cw, sw = dev(p["cw"]), dev(p["sw"])
    gw = dev(np.array([p["gw"]], np.float32))
    y = empty((M, N), np.float32)
    xd = dev(x)
    sel = torch.from_numpy(rows).cuda()
    if route == dm.ROUTE_INT8:
        q, s = empty((M, K), np.int8), empty((M,), np.float32)
        dm.hadamard_quant_int8(xd, q, s)
        dm.qgemm_int8(q, s, dev(p["qw"]), dev(p["sw_row"]), y)
        torch.cuda.synchronize()
        q0, s0 = orc.quant_int8(x)
        assert np.array_equal(host(q), q0) and np.array_equal(host(s).view(np.uint32), s0.view(np.uint32))
        _, y0 = orc.gemm_int8(q0, s0, p["qw"], p["sw_row"], rows=rows)
        assert np.array_equal(host(y[sel]).view(np.uint32), y0.view(np.uint32))
    else:
        c, sc, g = empty((M, K // 2), np.uint8), empty((M, K // 16), np.uint8), torch.zeros(1, device="cuda")
        dm.hadamard_quant_nvfp4(xd, c, sc, g, ws)
        dm.qgemm_nvfp4(c, sc, g, cw, sw, gw, y)
        torch.cuda.synchronize()
        c0, sc0, g0 = orc.quant_nvfp4(x)
        assert np.array_equal(host(c), c0) and np.array_equal(host(sc), sc0) and float(host(g)[0]) == g0
        y0, b0 = orc.gemm_nvfp4(c0, sc0, g0, p["cw"], p["sw"], p["gw"], rows=rows)
        assert np.all(np.abs(host(y[sel]).astype(np.float64) - y0) <= 1e-5 * b0)


def test_tiny_config_end_to_end(orc):
    """The tiny configuration (256 tokens x 256, four outlier channels x50,
    a 256 x 256 N(0, 1/256) weight): Gamma of a random residual block and the
    route; both quantized linears on every output row, the INT8 one through
    the one-launch quantizer with the weight conversion; a TDC refresh of the
    block and a skip from its cached delta."""
    require_gpu()
    say("tiny config end to end")
    cfg = wl.TINY
    M, K = cfg.M, cfg.hidden
    N = cfg.linears[0].N
    rng = np.random.default_rng(cfg.seeds[0])
    x = wl.activations(rng, M, K)
    assert wl.n_outlier_channels(K) == 4
    x_out = wl.residual_block_output(rng, x, K)
    w = wl.weight(rng, N, K)
    ws = dm.new_workspace(dm.OP_QUANT_NVFP4)
    s = torch.zeros(2, dtype=torch.float64, device="cuda")
    dm.gamma_sums(dev(x), dev(x_out), s, ws)
    torch.cuda.synchronize()
    s0 = orc.gamma_sums(x, x_out)
    assert np.all(np.abs(host(s) - s0) <= 1e-6 * s0)
    gam = s0[0] / s0[1]
    for tau in (0.5 * gam, 2.0 * gam):   # one threshold per route
        r = dm.gate_and_route(host(s), [1.0], [0.0], tau)[2]
        assert np.array_equal(r, orc.route(s0, [1.0], [0.0], tau)[2])
    p = orc.prep_weight(w)
    # INT8 route: activations and the NVFP4 -> INT8 weight in one launch
    q, sa = empty((M, K), np.int8), empty((M,), np.float32)
    qw, swr = empty((N, K), np.int8), empty((N,), np.float32)
    dm.hadamard_quant_int8_w8(dev(x), q, sa, dev(p["cw"]), dev(p["sw"]), dev(np.array([p["gw"]], np.float32)),
                              qw, swr)
    y8 = empty((M, N), np.float32)
    dm.qgemm_int8(q, sa, qw, swr, y8)
    # NVFP4 route
    c, sc, g = empty((M, K // 2), np.uint8), empty((M, K // 16), np.uint8), torch.zeros(1, device="cuda")
    dm.hadamard_quant_nvfp4(dev(x), c, sc, g, ws)
    y4 = empty((M, N), np.float32)
    dm.qgemm_nvfp4(c, sc, g, dev(p["cw"]), dev(p["sw"]), dev(np.array([p["gw"]], np.float32)), y4)
    torch.cuda.synchronize()
    q0, s0a = orc.quant_int8(x)
    assert np.array_equal(host(q), q0) and np.array_equal(host(sa).view(np.uint32), s0a.view(np.uint32))
    assert np.array_equal(host(qw), p["qw"]) and np.array_equal(host(swr).view(np.uint32),
                                                                p["sw_row"].view(np.uint32))
    _, y80 = orc.gemm_int8(q0, s0a, p["qw"], p["sw_row"])
    assert np.array_equal(host(y8).view(np.uint32), y80.view(np.uint32))
    c0, sc0, g0 = orc.quant_nvfp4(x)
    assert np.array_equal(host(c), c0) and np.array_equal(host(sc), sc0) and float(host(g)[0]) == g0
    y40, b0 = orc.gemm_nvfp4(c0, sc0, g0, p["cw"], p["sw"], p["gw"])
    assert np.all(np.abs(host(y4).astype(np.float64) - y40) <= 1e-5 * b0)
    # TDC: refresh caches delta = out - in, then a skip rebuilds out from it
    delta = torch.zeros(M * K, dtype=torch.int16, device="cuda")
    sums = torch.zeros(4, dtype=torch.float64, device="cuda")
    dm.tdc_step(dm.TDC_REFRESH, dev(x).view(-1), dev(x_out).view(-1), delta, False, sums,
                dm.new_workspace(dm.OP_TDC))
    out = torch.empty(M * K, dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    d0 = np.zeros(M * K, np.uint16)
    t0 = orc.tdc_refresh(x.ravel(), x_out.ravel(), d0, False)
    assert np.array_equal(host(delta, np.uint16), d0)
    assert np.all(np.abs(host(sums)[:2] - t0[:2]) <= 1e-6 * np.abs(t0[:2]))
    dm.tdc_step(dm.TDC_SKIP, dev(x).view(-1), out, delta, True)
    torch.cuda.synchronize()
    assert np.array_equal(host(out, np.uint16), orc.tdc_skip(x.ravel(), d0))


def test_cogvideox5b_routing_and_linears(orc):
    require_gpu()
    cfg = wl.COGVIDEOX_5B
    M, H = cfg.M, cfg.hidden
    alpha = np.full(4, wl.ROUTER_5B["alpha"])
    beta = np.full(4, wl.ROUTER_5B["beta"])
    tau = wl.ROUTER_5B["tau"]
    ws = dm.new_workspace(dm.OP_GAMMA)
    routes = []
    for b, seed in enumerate(cfg.seeds):
        say(f"5B-like block {b}: gamma + route")
        rng = np.random.default_rng(seed)
        x_in = wl.activations(rng, M, H)
        x_out = wl.perturbed_output(rng, x_in, wl.GAMMA_TARGETS_5B[b])
        s = torch.zeros(2, dtype=torch.float64, device="cuda")
        dm.gamma_sums(dev(x_in), dev(x_out), s, ws)
        torch.cuda.synchronize()
        s0 = orc.gamma_sums(x_in, x_out)
        assert np.all(np.abs(host(s) - s0) <= 1e-6 * s0)
        g, e, r = dm.gate_and_route(host(s), alpha, beta, tau)
        _, e0, r0 = orc.route(s0, alpha, beta, tau)
        assert np.array_equal(r, r0)
        assert abs(g - wl.GAMMA_TARGETS_5B[b]) < 0.01       # the synthetic Gamma hits its target
        routes.append(int(r[0]))
    assert routes == [dm.ROUTE_NVFP4, dm.ROUTE_INT8, dm.ROUTE_NVFP4, dm.ROUTE_INT8]
    # each route on every 5B linear shape, full token count, sampled GEMM rows
    for li, lin in enumerate(cfg.linears):
        for route in (dm.ROUTE_NVFP4, dm.ROUTE_INT8):
            say(f"5B-like linear {lin.name} N={lin.N} K={lin.K} route={route}")
            _linear_parity(orc, np.random.default_rng(100 + 10 * li + route), M, lin.N, lin.K,
                           route, _rows(M, 1481))


@pytest.mark.parametrize("route", [0, 1])
def test_1080p_ffn_up_linear(orc, route):
    require_gpu()
    M, N, K = wl.M_1080P, 12288, 3072
    say(f"1080p-like ffn_up M={M} N={N} K={K} route={route}")
    _linear_parity(orc, np.random.default_rng(1080 + route), M, N, K, route, _rows(M, 8861))


def test_cogvideox2b_linears(orc):
    require_gpu()
    cfg = wl.COGVIDEOX_2B
    for li, lin in enumerate(cfg.linears):
        for route in (dm.ROUTE_NVFP4, dm.ROUTE_INT8):
            say(f"2B-like linear {lin.name} N={lin.N} K={lin.K} route={route}")
            _linear_parity(orc, np.random.default_rng(200 + 10 * li + route), cfg.M, lin.N, lin.K,
                           route, _rows(cfg.M, 1481))


@pytest.mark.parametrize("route", [0, 1])
def test_1080p_ffn_down_linear(orc, route):
    require_gpu()
    M, N, K = wl.M_1080P, 3072, 12288
    say(f"1080p-like ffn_down M={M} N={N} K={K} route={route}")
    _linear_parity(orc, np.random.default_rng(1090 + route), M, N, K, route, _rows(M, 8861))


def _tail_tile_rows(M, N, nk, splits_from_k=True):
    """Rows of the m-tiles that hold tail tiles of a split launch: the logical
    tile ids full .. tiles-1 in the library's grouped order (8 tile rows per
    group, down a group's rows before moving right)."""
    tm, tn = -(-M // 256), -(-N // 256)
    tiles = tm * tn
    tail = tiles % 256
    s = min(256 // tail, nk) if tail else 0
    if not splits_from_k or tail == 0 or s < 2:
        return np.zeros(0, np.int64)
    mt = set()
    for pid in range(tiles - tail, tiles):
        g, in_group = divmod(pid, 8 * tn)
        rows_in_group = min(tm - 8 * g, 8)
        mt.add(8 * g + in_group % rows_in_group)
    return np.concatenate([np.arange(256 * t, min(256 * t + 256, M)) for t in sorted(mt)])


def _bench_launch_parity(orc, cfg, li, route, seed, every):
    """One linear of cfg launched as the benchmark does: the *_ex GEMMs with
    the full GEMM workspace (tail split) and bf16 output.  The row sample
    takes every 37th row of the m-tiles that hold split tail tiles, plus every
    `every`-th row and the last 3."""
    M = cfg.M
    lin = cfg.linears[li]
    N, K = lin.N, lin.K
    # stages of the split plan: INT8 128 K elements; NVFP4 256, plus the
    # closing half stage when K % 256 == 128
    nk = K // 128 if route == dm.ROUTE_INT8 else K // 256 + (1 if K % 256 else 0)
    tail = _tail_tile_rows(M, N, nk, route != dm.ROUTE_INT8 or K >= 4096)
    rows = np.unique(np.concatenate([tail[::37], np.arange(0, M, every), np.arange(M - 3, M)]))
    say(f"{cfg.name} {lin.name} M={M} N={N} K={K} route={route} bench launch, "
        f"{len(tail)} tail-tile rows, {len(rows)} rows checked")
    rng = np.random.default_rng(seed)
    x = wl.activations(rng, M, K)
    p = orc.prep_weight(wl.weight(rng, N, K))
    ws = dm.new_workspace(dm.OP_GEMM, "cuda", M, N)
    y = empty((M, N), np.uint16)
    sel = torch.from_numpy(rows).cuda()
    if route == dm.ROUTE_INT8:
        q0, s0 = orc.quant_int8(x)
        del x
        dm.qgemm_int8_ex(dev(q0), dev(s0), dev(p["qw"]), dev(p["sw_row"]), y, 0, ws, dm.OUT_BF16)
        torch.cuda.synchronize()
        _, y0 = orc.gemm_int8(q0, s0, p["qw"], p["sw_row"], rows=rows)
        assert np.array_equal(host(y[sel], np.uint16), wl.to_bf16_bits(y0))
    else:
        c0, sc0, g0 = orc.quant_nvfp4(x)
        del x
        dm.qgemm_nvfp4_ex(dev(c0), dev(sc0), dev(np.array([g0], np.float32)), dev(p["cw"]),
                          dev(p["sw"]), dev(np.array([p["gw"]], np.float32)), y, 0, ws, dm.OUT_BF16)
        torch.cuda.synchronize()
        y0, b0 = orc.gemm_nvfp4(c0, sc0, g0, p["cw"], p["sw"], p["gw"], rows=rows)
        yb = wl.bf16_bits_to_f32(host(y[sel], np.uint16)).astype(np.float64)
        assert np.all(np.abs(yb - y0) <= 1e-5 * b0 + 2.0 ** -8 * np.abs(y0))


@pytest.mark.parametrize("route", [0, 1])
@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_1080p_linears_bench_launch(orc, li, route):
    """Every 1080p-like linear on both routes, launched as the benchmark does.
    NVFP4 qkv, out and ffn_down and INT8 ffn_down split a 128-tile tail in
    two (the two-way fixup); INT8 below K = 4096 and ffn_up (no tail) run
    unsplit."""
    require_gpu()
    _bench_launch_parity(orc, wl.VIDEO_1080P, li, route, 1100 + 10 * li + route, 1499)


@pytest.mark.parametrize("route", [0, 1])
@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_2b_linears_bench_launch(orc, li, route):
    """Every 2B-like linear on both routes, launched as the benchmark does.
    The NVFP4 K = 1920 linears run 256-element stages and the closing half
    stage, their tails split 3 or 4 ways; INT8 splits only ffn_down
    (K = 7680)."""
    require_gpu()
    _bench_launch_parity(orc, wl.COGVIDEOX_2B, li, route, 1300 + 10 * li + route, 997)


@pytest.mark.parametrize("li", [0, 1, 2, 3])
def test_w4a8_chain_5b(orc, li):
    """The INT8 route with only the NVFP4 weight kept, as the benchmark runs
    it: the weight converted to INT8 into a scratch buffer right before the
    GEMM (dmpq_weight_int8_from_nvfp4), then the _ex GEMM with the full
    workspace and fp32 output -- bit-exact against the oracle's conversion
    followed by its INT8 GEMM, on a row sample of the 5B-like shapes."""
    require_gpu()
    cfg = wl.COGVIDEOX_5B
    lin = cfg.linears[li]
    M, N, K = cfg.M, lin.N, lin.K
    say(f"W4A8 chain 5B-like {lin.name} M={M} N={N} K={K}")
    rng = np.random.default_rng(400 + li)
    x = wl.activations(rng, M, K)
    w = wl.weight(rng, N, K)
    p = orc.prep_weight(w)
    q0, s0 = orc.quant_int8(x)
    qw0, sw0 = orc.w8_from_nvfp4(p["cw"], p["sw"], p["gw"])
    rows = _rows(M, 997)
    _, y0 = orc.gemm_int8(q0, s0, qw0, sw0, rows=rows)
    qw, swr = empty((N, K), np.int8), empty((N,), np.float32)
    dm.weight_int8_from_nvfp4(dev(p["cw"]), dev(p["sw"]), dev(np.array([p["gw"]], np.float32)), qw, swr)
    y = empty((M, N), np.float32)
    dm.qgemm_int8_ex(dev(q0), dev(s0), qw, swr, y, 0, dm.new_workspace(dm.OP_GEMM, "cuda", M, N),
                     dm.OUT_F32)
    torch.cuda.synchronize()
    assert np.array_equal(host(qw), qw0) and np.array_equal(host(swr).view(np.uint32), sw0.view(np.uint32))
    sel = torch.from_numpy(rows).cuda()
    assert np.array_equal(host(y[sel]).view(np.uint32), y0.view(np.uint32))
