"""The allocation-free NVFP4 quantizer (dmpq_hadamard_quant_nvfp4_noalloc,
for callers that cannot allocate device memory) against the workspace entry
point it varies: bit-identical codes, block scales and tensor scale on two
calls in a row, the second with a smaller input, so the second call runs on
a scratch array that still holds the first call's partial maxima.  Also
against the oracle, and its argument errors."""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, empty, host, require_gpu, say

pytestmark = pytest.mark.gpu


def _run(fn, x, flags, *ws):
    M, K = x.shape
    c, s = empty((M, K // 2), np.uint8), empty((M, K // 16), np.uint8)
    g = torch.full((1,), -1.0, device="cuda")
    c.fill_(0xAB)
    s.fill_(0xCD)
    fn(x, c, s, g, *ws, flags=flags)
    torch.cuda.synchronize()
    return host(c), host(s), np.float32(host(g)[0])


@pytest.mark.parametrize("flags", [0, dm.NO_HADAMARD])
def test_noalloc_matches_workspace_call(orc, flags):
    require_gpu()
    ws = dm.new_workspace(dm.OP_QUANT_NVFP4)
    # the larger call first (512 first-pass partials, the cap), then a smaller one
    # whose tensor amax is lower, so stale partials would show in g
    for (M, K), seed, scale in (((4096, 3072), 70, 50.0), ((37, 208), 71, 1.0)):
        say(f"noalloc nvfp4 quant M={M} K={K} flags={flags}")
        xh = workloads.activations(np.random.default_rng(seed), M, K, outlier_scale=scale)
        x = dev(xh).view(M, K)
        a = _run(dm.hadamard_quant_nvfp4_noalloc, x, flags)
        b = _run(dm.hadamard_quant_nvfp4, x, flags, ws)
        assert a[2].view(np.uint32) == b[2].view(np.uint32)
        assert np.array_equal(a[1], b[1]) and np.array_equal(a[0], b[0])
        c0, s0, g0 = orc.quant_nvfp4(xh, flags)
        assert a[2].view(np.uint32) == np.float32(g0).view(np.uint32)
        assert np.array_equal(a[1], s0) and np.array_equal(a[0], c0)


def test_noalloc_empty_and_errors():
    require_gpu()
    say("noalloc nvfp4 quant: empty input and argument errors")
    g = torch.full((1,), -1.0, device="cuda")
    dm.hadamard_quant_nvfp4_noalloc(empty((0, 64), np.uint16), empty((0, 32), np.uint8),
                                    empty((0, 4), np.uint8), g)
    torch.cuda.synchronize()
    assert float(g[0]) == 0.0
    x = empty((4, 64), np.uint16)
    c, s = empty((4, 32), np.uint8), empty((4, 4), np.uint8)
    with pytest.raises(dm.DmpqError) as ei:
        dm.hadamard_quant_nvfp4_noalloc(x, c, s, g, flags=dm.AMAX_GIVEN)
    assert ei.value.status == 4 and "AMAX_GIVEN" in str(ei.value)
    with pytest.raises(dm.DmpqError) as ei:
        dm.hadamard_quant_nvfp4_noalloc(x, c, s, g, flags=8)
    assert ei.value.status == 1
