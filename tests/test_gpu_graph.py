"""GPU: the library's calls captured in a HIP graph and replayed.

The entry points allocate nothing (workspaces are the caller's; the NVFP4
quantizer also has a form without one), record no memsets and never
synchronize, so a caller may capture them.  One NVFP4-routed and one
INT8-routed linear (quantize, convert the weight, GEMM with the tail-split
workspace) are captured in one graph; each replay follows an eager change of
the input and a synchronization, and its outputs must equal, bit for bit, an
eager run of the same calls on the same input.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, require_gpu, say

pytestmark = pytest.mark.gpu


def test_graph_replay_of_two_linears(orc):
    require_gpu()
    say("graph capture and replay: NVFP4 and INT8 linears")
    rng = np.random.default_rng(123)
    M, K, N = 700, 768, 520
    xs = [dev(workloads.activations(rng, M, K)) for _ in range(4)]
    p = orc.prep_weight(workloads.weight(rng, N, K))
    cw, sw, gw = dev(p["cw"]), dev(p["sw"]), dev(np.array([p["gw"]], np.float32))

    x = torch.empty_like(xs[0])
    c = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    g = torch.empty(1, device="cuda")
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty(M, device="cuda")
    qw = torch.empty((N, K), dtype=torch.int8, device="cuda")
    swr = torch.empty(N, device="cuda")
    y4 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y8 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws4 = dm.new_workspace(dm.OP_GEMM, "cuda", M, N)
    ws8 = dm.new_workspace(dm.OP_GEMM, "cuda", M, N)

    def linears():
        dm.hadamard_quant_nvfp4_noalloc(x, c, sc, g)
        dm.qgemm_nvfp4_ex(c, sc, g, cw, sw, gw, y4, 0, ws4)
        dm.hadamard_quant_int8(x, qa, sa)
        dm.weight_int8_from_nvfp4(cw, sw, gw, qw, swr)
        dm.qgemm_int8_ex(qa, sa, qw, swr, y8, 0, ws8)

    def eager(xi):
        x.copy_(xi)
        linears()
        torch.cuda.synchronize()
        return y4.clone(), y8.clone(), c.clone(), g.clone()

    want = [eager(xi) for xi in xs[1:]]  # also sets up every kernel before the capture

    graph = torch.cuda.CUDAGraph()
    x.copy_(xs[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        linears()
    torch.cuda.synchronize()

    for r, xi in enumerate(xs[1:]):
        y4.zero_()
        y8.zero_()
        x.copy_(xi)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        w4, w8, wc, wg = want[r]
        assert torch.equal(c, wc) and torch.equal(g, wg), r
        assert torch.equal(y4.view(torch.int16), w4.view(torch.int16)), r
        assert torch.equal(y8.view(torch.int16), w8.view(torch.int16)), r


def test_graph_replay_of_a_routed_block(orc):
    """A whole block as the bench's --graph mode captures it: four linears on
    mixed routes (NVFP4 through the workspace quantizer, INT8 through the
    one-launch quantizer with the weight conversion), each GEMM with the
    tail-split workspace, then the block's TDC refresh.  Three replays, each
    after an eager change of the inputs and of the cached delta, equal eager
    runs bit for bit: outputs, codes, the new delta and the refresh sums."""
    require_gpu()
    say("graph capture and replay: a routed block with its TDC refresh")
    rng = np.random.default_rng(321)
    M, H, F = 600, 256, 512
    shapes = [(3 * H, H), (H, H), (F, H), (H, F)]  # (N, K): qkv, out, ffn_up, ffn_down
    routes = [dm.ROUTE_NVFP4, dm.ROUTE_INT8, dm.ROUTE_NVFP4, dm.ROUTE_INT8]
    lins = []
    for N, K in shapes:
        p = orc.prep_weight(workloads.weight(rng, N, K))
        lins.append(dict(N=N, K=K, cw=dev(p["cw"]), sw=dev(p["sw"]), gw=dev(np.array([p["gw"]], np.float32)),
                         x=torch.empty((M, K), dtype=torch.int16, device="cuda"),
                         y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                         ws=dm.new_workspace(dm.OP_GEMM, "cuda", M, N)))
    qb = {K: dict(q=torch.empty((M, K), dtype=torch.int8, device="cuda"), s=torch.empty(M, device="cuda"),
                  c=torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                  sc=torch.empty((M, K // 16), dtype=torch.uint8, device="cuda"),
                  g=torch.empty(1, device="cuda")) for K in (H, F)}
    qw = torch.empty(max(N * K for N, K in shapes), dtype=torch.int8, device="cuda")
    swr = torch.empty(max(N for N, _ in shapes), device="cuda")
    wsq = dm.new_workspace(dm.OP_QUANT_NVFP4)
    wst = dm.new_workspace(dm.OP_TDC)
    x_in = torch.empty(M * H, dtype=torch.int16, device="cuda")
    x_out = torch.empty(M * H, dtype=torch.int16, device="cuda")
    delta = torch.empty(M * H, dtype=torch.int16, device="cuda")
    sums = torch.zeros(4, dtype=torch.float64, device="cuda")

    def block():
        for L, route in zip(lins, routes):
            b = qb[L["K"]]
            if route == dm.ROUTE_INT8:
                w8 = qw[:L["N"] * L["K"]].view(L["N"], L["K"])
                dm.hadamard_quant_int8_w8(L["x"], b["q"], b["s"], L["cw"], L["sw"], L["gw"], w8, swr[:L["N"]])
                dm.qgemm_int8_ex(b["q"], b["s"], w8, swr[:L["N"]], L["y"], 0, L["ws"])
            else:
                dm.hadamard_quant_nvfp4(L["x"], b["c"], b["sc"], b["g"], wsq)
                dm.qgemm_nvfp4_ex(b["c"], b["sc"], b["g"], L["cw"], L["sw"], L["gw"], L["y"], 0, L["ws"])
        dm.tdc_step(dm.TDC_REFRESH, x_in, x_out, delta, True, sums, wst)

    def inputs(seed):
        r = np.random.default_rng(seed)
        xs = [dev(workloads.activations(r, M, L["K"])) for L in lins]
        xi = workloads.activations(r, M, H)
        xo = workloads.perturbed_output(r, xi, 0.2)
        d0 = workloads.perturbed_output(r, xi, 0.1)
        return xs, dev(xi).view(-1), dev(xo).view(-1), dev(d0).view(-1)

    def load(inp):
        xs, xi, xo, d0 = inp
        for L, xv in zip(lins, xs):
            L["x"].copy_(xv)
        x_in.copy_(xi)
        x_out.copy_(xo)
        delta.copy_(d0)

    def outputs():
        return ([L["y"].clone() for L in lins], qb[H]["c"].clone(), qb[F]["q"].clone(), delta.clone(),
                sums.clone())

    feeds = [inputs(s) for s in (11, 12, 13, 14)]
    want = []
    for inp in feeds[1:]:  # eager runs (they also set up every kernel before the capture)
        load(inp)
        block()
        torch.cuda.synchronize()
        want.append(outputs())
    graph = torch.cuda.CUDAGraph()
    load(feeds[0])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        block()
    torch.cuda.synchronize()
    for r, inp in enumerate(feeds[1:]):
        for L in lins:
            L["y"].zero_()
        load(inp)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ys, c, q, d, s = outputs()
        wy, wc, wq, wd, wsum = want[r]
        for a, b in zip(ys, wy):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), r
        assert torch.equal(c, wc) and torch.equal(q, wq), r
        assert torch.equal(d, wd), r
        assert torch.equal(s, wsum), r
