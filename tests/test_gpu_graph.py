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
