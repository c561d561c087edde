"""GPU: the router calibration of the proxy DiT.

Over always-refresh steps, each linear's NVFP4 relative L1 error (against the
BF16 GEMM) is paired with the block's Gamma of the previous step and a line
is fitted per linear.  Checked: each measured error equals the oracle's sums
on the same two GPU outputs; the NVFP4 and BF16 outputs the error is built
from agree with the oracle's GEMMs; the fit is finite and its predictions
route the calibration samples the way a threshold between them implies.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
from dynamic_mixed_precision_amd.calibrate import ErrorProbe, fit_router
from dynamic_mixed_precision_amd.schedule import TdcScheduler
from gpu_util import host, require_gpu, say
from proxy_dit import ProxyDiT

pytestmark = pytest.mark.gpu


def _bits(t):
    return host(t.contiguous().view(torch.int16), np.uint16).reshape(t.shape)


def test_router_calibration_on_proxy_dit(orc):
    require_gpu()
    M, H, NB, T = 512, 256, 6, 5
    say(f"router calibration on the proxy DiT M={M} H={H} blocks={NB} steps={T}")
    dit = ProxyDiT(M, H, NB, seed=12)
    sched = TdcScheduler(NB, M * H, [1.0, 1.0], [0.0, 0.0], np.inf, 0.0, 0.0)
    probe = ErrorProbe(M, H, H)
    gam, err = [], []
    checked = 0
    z = dit.x0
    for t in range(T):
        sched.begin_step()
        x = z
        for i in range(NB):
            st = sched.blocks[i].state
            lin1, lin2 = dit.blocks[i]
            if st.gamma_valid:
                e1 = probe(x, lin1.w, lin1.cw, lin1.sw, lin1.gw)
                if checked < 3:
                    torch.cuda.synchronize()
                    s_ref = orc.gamma_sums(_bits(probe.y_ref).ravel(), _bits(probe.y_q).ravel())
                    assert abs(e1 - s_ref[0] / s_ref[1]) <= 1e-6 * e1
                    xh = _bits(x)
                    yb, bb = orc.gemm_bf16(xh, _bits(lin1.w))
                    yr = host(probe.y_ref.view(torch.bfloat16).float()).astype(np.float64)
                    assert np.all(np.abs(yr - yb) <= 1e-5 * bb + 2.0 ** -8 * np.abs(yb))
                    c, sc, g = orc.quant_nvfp4(xh)
                    yn, bn = orc.gemm_nvfp4(c, sc, g, host(lin1.cw), host(lin1.sw), float(host(lin1.gw)[0]))
                    yq = host(probe.y_q.view(torch.bfloat16).float()).astype(np.float64)
                    assert np.all(np.abs(yq - yn) <= 1e-5 * bn + 2.0 ** -8 * np.abs(yn))
                    checked += 1
                gam.append(st.gamma)
                out = dit.block_forward(i, x, np.array([dm.ROUTE_BF16, dm.ROUTE_BF16]))
                # the second linear's input is GELU of the first linear's BF16 output
                y1 = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
                dm.gemm_bf16(x.view(torch.int16), lin1.w.view(torch.int16), y1, dm.OUT_BF16)
                h = torch.nn.functional.gelu(y1.float()).to(torch.bfloat16)
                e2 = probe(h, lin2.w, lin2.cw, lin2.sw, lin2.gw)
                err.append([e1, e2])
            else:
                out = dit.block_forward(i, x, np.array([dm.ROUTE_BF16, dm.ROUTE_BF16]))
            sched.refresh(i, x, out)
            x = out
        z = dit.drift(z)
    gam = np.array(gam)
    err = np.array(err)
    alpha, beta, rms = fit_router(gam, err)
    say(f"  samples={len(gam)} gamma {gam.min():.3g}..{gam.max():.3g} "
        f"error l1 {err[:, 0].min():.3g}..{err[:, 0].max():.3g} l2 {err[:, 1].min():.3g}..{err[:, 1].max():.3g}")
    say(f"  alpha={alpha} beta={beta} rms={rms}")
    assert checked == 3 and len(gam) == NB * (T - 1)
    assert np.all(np.isfinite(alpha)) and np.all(np.isfinite(beta))
    assert np.all((err > 0) & (err < 1))
    # a threshold at the median prediction splits the samples through the router
    pred = gam[:, None] * alpha + beta
    tau = float(np.median(pred[:, 0]))
    for k in range(len(gam)):
        _, e, r = dm.gate_and_route(np.array([gam[k], 1.0]), alpha, beta, tau)
        assert np.allclose(e, pred[k], rtol=1e-12)
        assert r[0] == (dm.ROUTE_INT8 if pred[k, 0] > tau else dm.ROUTE_NVFP4)
