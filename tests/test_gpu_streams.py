"""GPU: calls on two streams at once, each with its own workspaces.

The header allows concurrent calls on different streams as long as they do
not share a workspace.  Two independent sets of a block's calls (the NVFP4
quantizer and split GEMM, the INT8 quantizer with the weight conversion and
split GEMM, Gamma's sums, the TDC refresh and the PDR outlier count) are
enqueued alternately on two streams, so their kernels can overlap on the
device.  Every output must equal, bit for bit, the same calls run one after
another on one stream: a library state shared between calls (a static
buffer, a counter, a finalize slot) would show up as a difference.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, require_gpu, say

pytestmark = pytest.mark.gpu


def _lane(orc, seed, M, K, N):
    rng = np.random.default_rng(seed)
    p = orc.prep_weight(workloads.weight(rng, N, K))
    x = dev(workloads.activations(rng, M, K))
    xi_bits = workloads.activations(rng, M, K)
    L = dict(x=x, cw=dev(p["cw"]), sw=dev(p["sw"]), gw=dev(np.array([p["gw"]], np.float32)),
             xi=dev(xi_bits).view(-1),
             xo=dev(workloads.perturbed_output(rng, xi_bits, 0.2)).view(-1),
             d0=dev(workloads.perturbed_output(rng, xi_bits, 0.1)).view(-1))
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    L.update(c=torch.empty((M, K // 2), **u8), sc=torch.empty((M, K // 16), **u8),
             g=torch.empty(1, **f32), q=torch.empty((M, K), dtype=torch.int8, device="cuda"),
             s=torch.empty(M, **f32), qw=torch.empty((N, K), dtype=torch.int8, device="cuda"),
             swr=torch.empty(N, **f32),
             y4=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
             y8=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
             delta=torch.empty(M * K, dtype=torch.int16, device="cuda"),
             gsum=torch.empty(2, dtype=torch.float64, device="cuda"),
             tsum=torch.empty(4, dtype=torch.float64, device="cuda"),
             cnt=torch.empty(1, dtype=torch.float64, device="cuda"),
             wsq=dm.new_workspace(dm.OP_QUANT_NVFP4, "cuda", M, K),
             wsg4=dm.new_workspace(dm.OP_GEMM, "cuda", M, N),
             wsg8=dm.new_workspace(dm.OP_GEMM, "cuda", M, N), wsgam=dm.new_workspace(dm.OP_GAMMA),
             wst=dm.new_workspace(dm.OP_TDC), wso=dm.new_workspace(dm.OP_OUTLIER))
    return L


def _ops(L, st):
    """The block's calls in order, each a closure enqueued on stream st."""
    return [
        lambda: L["delta"].copy_(L["d0"]),
        lambda: dm.hadamard_quant_nvfp4(L["x"], L["c"], L["sc"], L["g"], L["wsq"], stream=st),
        lambda: dm.qgemm_nvfp4_ex(L["c"], L["sc"], L["g"], L["cw"], L["sw"], L["gw"], L["y4"], 0,
                                  L["wsg4"], stream=st),
        lambda: dm.hadamard_quant_int8_w8(L["x"], L["q"], L["s"], L["cw"], L["sw"], L["gw"], L["qw"],
                                          L["swr"], stream=st),
        lambda: dm.qgemm_int8_ex(L["q"], L["s"], L["qw"], L["swr"], L["y8"], 0, L["wsg8"], stream=st),
        lambda: dm.gamma_sums(L["xi"], L["xo"], L["gsum"], L["wsgam"], stream=st),
        lambda: dm.tdc_step(dm.TDC_REFRESH, L["xi"], L["xo"], L["delta"], True, L["tsum"], L["wst"],
                            stream=st),
        lambda: dm.outlier_count(L["x"], 4.0, L["cnt"], L["wso"], stream=st),
    ]


_OUT = ("c", "sc", "g", "q", "s", "qw", "swr", "y4", "y8", "delta", "gsum", "tsum", "cnt")


def _snapshot(L):
    return {k: L[k].clone() for k in _OUT}


def _clear(L):
    for k in _OUT:
        L[k].zero_()


@pytest.mark.parametrize("M,K,N", [(1000, 768, 520), (2300, 4096, 1100)])
def test_two_streams_match_one(orc, M, K, N):
    require_gpu()
    say(f"two streams against one: M={M} K={K} N={N}")
    lanes = [_lane(orc, 40 + i, M, K, N) for i in range(2)]
    main = torch.cuda.current_stream()
    want = []
    for L in lanes:  # one after another on one stream
        _clear(L)
        for op in _ops(L, main):
            op()
        torch.cuda.synchronize()
        want.append(_snapshot(L))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    for r in range(3):
        for L in lanes:
            _clear(L)
        torch.cuda.synchronize()
        per_lane = [_ops(L, s) for L, s in zip(lanes, streams)]
        for step in range(len(per_lane[0])):  # alternate the two streams call by call
            for i, s in enumerate(streams):
                with torch.cuda.stream(s):
                    per_lane[i][step]()
        torch.cuda.synchronize()
        for i, L in enumerate(lanes):
            for k in _OUT:
                a, b = L[k], want[i][k]
                if a.dtype == torch.bfloat16:
                    a, b = a.view(torch.int16), b.view(torch.int16)
                assert torch.equal(a, b), (r, i, k)
