"""GPU parity of the full hot path under the Temporal Delta Cache schedule.

Proxy DiT (residual blocks x + W2 GELU(W1 x), hidden H; each timestep runs
the blocks on a drifting latent z_t = z_{t-1} + 0.02 N(0,1)).  Thresholds come from a calibration pass that
always refreshes: tau = median Gamma (alpha = 1, beta = 0, so about half the
blocks route to INT8), eps_sim = median d, delta_acc = 2.5 * median d.

* Lockstep (small): every contract call the GPU makes is recomputed by the
  oracle from the GPU's own inputs: quantizers bit-exact, GEMMs within
  1e-5 * B (plus bf16 output rounding), TDC sums within 1e-6, cached delta
  and skip outputs bit-exact, and every routing / skip decision equal to the
  oracle's on the oracle's sums (except inside the 1e-5 tie band, counted).
* Full size (42 blocks x 50 steps, 17776 tokens x 1920): host decisions
  mirrored by the oracle on the same sums, plus deep checks of sampled
  refresh and skip events.
* Lockstep with Purified Delta Refresh: every refresh first counts the block
  input's outliers (kappa = 4) and forces the block's linears to BF16 when
  the ratio exceeds rho = the median ratio seen in calibration; the count and
  the decision match the oracle's, and forced blocks run the BF16 GEMM,
  checked against the oracle.
"""
import math

import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
from dynamic_mixed_precision_amd.schedule import TdcScheduler
from gpu_util import host, require_gpu, say
from proxy_dit import ProxyDiT

pytestmark = pytest.mark.gpu

TIE = 1e-5


def _bits(t):
    return host(t.contiguous().view(torch.int16), np.uint16).reshape(t.shape)


def _calibrate(dit, steps=3):
    """Always refresh (eps_sim = 0); all NVFP4 unless Gamma is missing."""
    NB = len(dit.blocks)
    sched = TdcScheduler(NB, dit.M * dit.H, [1.0, 1.0], [0.0, 0.0], math.inf, 0.0, 0.0)
    z = dit.x0
    for _ in range(steps):
        sched.begin_step()
        x = z
        for i in range(NB):
            r = sched.routes(i)[2]
            out = dit.block_forward(i, x, r)
            sched.refresh(i, x, out)
            x = out
        z = dit.drift(z)
    sched.begin_step()
    gam = [b.state.gamma for b in sched.blocks]
    ds = [b.state.d for b in sched.blocks]
    med_d = float(np.median(ds))
    return float(np.median(gam)), med_d, 2.5 * med_d


def _in_tie(v, thr):
    return abs(v - thr) <= TIE * max(abs(thr), 1e-12)


def _calibrate_pdr(dit, kappa, steps=3):
    """Median outlier ratio of the block inputs over always-refresh steps."""
    NB = len(dit.blocks)
    ws = dm.new_workspace(dm.OP_OUTLIER)
    cnt = torch.zeros(1, dtype=torch.float64, device="cuda")
    ratios = []
    z = dit.x0
    for _ in range(steps):
        x = z
        for i in range(NB):
            dm.outlier_count(x, kappa, cnt, ws)
            ratios.append(float(cnt.item()) / x.numel())
            x = dit.block_forward(i, x, np.array([dm.ROUTE_INT8, dm.ROUTE_INT8]))
        z = dit.drift(z)
    return float(np.median(ratios)), ratios


class LinearChecker:
    """Hook of routed_linear: recompute quant + GEMM with the oracle."""

    def __init__(self, orc):
        self.orc = orc
        self.calls = {0: 0, 1: 0, 2: 0}

    def __call__(self, x, lin, route, qb, y):
        orc = self.orc
        torch.cuda.synchronize()
        xh = _bits(x)
        yb = _bits(y).astype(np.uint16)
        yf = torch.from_numpy(yb.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
        if route == dm.ROUTE_BF16:
            y_ref, bound = orc.gemm_bf16(xh, _bits(lin.w))
            assert np.all(np.abs(yf - y_ref) <= 1e-5 * bound + 2.0 ** -8 * np.abs(y_ref))
        elif route == dm.ROUTE_INT8:
            q, s = orc.quant_int8(xh)
            assert np.array_equal(host(qb.q), q) and np.array_equal(host(qb.s).view(np.uint32), s.view(np.uint32))
            _, y_ref = orc.gemm_int8(q, s, host(lin.qw), host(lin.swr))
            y32 = torch.from_numpy(y_ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(yb, y32)
        else:
            c, sc, g = orc.quant_nvfp4(xh)
            assert np.array_equal(host(qb.c), c) and np.array_equal(host(qb.sc), sc)
            assert np.float32(host(qb.g)[0]) == np.float32(g)
            y_ref, bound = orc.gemm_nvfp4(c, sc, g, host(lin.cw), host(lin.sw), float(host(lin.gw)[0]))
            assert np.all(np.abs(yf - y_ref) <= 1e-5 * bound + 2.0 ** -8 * np.abs(y_ref))
        self.calls[route] += 1


def test_proxy_schedule_lockstep(orc):
    require_gpu()
    M, H, NB, T = 512, 256, 6, 14
    say(f"proxy DiT lockstep M={M} H={H} blocks={NB} steps={T}")
    tau, eps, dacc = _calibrate(ProxyDiT(M, H, NB, seed=10))
    say(f"  calibrated tau={tau:.4g} eps_sim={eps:.4g} delta_acc={dacc:.4g}")
    dit = ProxyDiT(M, H, NB, seed=10)
    alpha, beta = np.array([1.0, 1.0]), np.array([0.0, 0.0])
    sched = TdcScheduler(NB, M * H, alpha, beta, tau, eps, dacc)
    mirror = [orc.tdc_new() for _ in range(NB)]
    mirror_sums2 = [None] * NB
    pending = [None] * NB
    checker = LinearChecker(orc)
    ties = 0
    skips = 0
    z = dit.x0
    for t in range(T):
        sched.begin_step()
        x = z
        for i in range(NB):
            if pending[i] is not None:
                orc.tdc_commit_refresh(mirror[i], pending[i])
                mirror_sums2[i] = pending[i][:2].copy()
                pending[i] = None
        for i in range(NB):
            st = mirror[i]
            skip = sched.decide(i)
            skip_o = orc.tdc_decide(st, eps, dacc)
            if st.n_refresh >= 2 and (_in_tie(st.d, eps) or _in_tie(st.acc + st.d, dacc)):
                ties += 1
            else:
                assert skip == skip_o, (t, i)
            xh = _bits(x)
            blk = sched.blocks[i]
            if skip:
                skips += 1
                d_before = _bits(blk.delta)
                out = torch.empty_like(x)
                sched.skip(i, x, out)
                torch.cuda.synchronize()
                assert np.array_equal(_bits(out).ravel(), orc.tdc_skip(xh.ravel(), d_before))
                orc.tdc_commit_skip(st)
            else:
                _, e, r = sched.routes(i)
                sums2 = mirror_sums2[i] if st.gamma_valid else None
                _, e_o, r_o = orc.route(sums2, alpha, beta, tau)
                for l in range(2):
                    if sums2 is not None and _in_tie(e_o[l], tau):
                        ties += 1
                    else:
                        assert r[l] == r_o[l], (t, i, l)
                out = dit.block_forward(i, x, r, hook=checker)
                d_ref = _bits(blk.delta).ravel().copy()
                dv = bool(blk.state.delta_valid)
                sched.refresh(i, x, out)
                torch.cuda.synchronize()
                s_ref = orc.tdc_refresh(xh.ravel(), _bits(out).ravel(), d_ref, dv)
                assert np.array_equal(_bits(blk.delta).ravel(), d_ref)
                s_gpu = host(blk.sums)
                assert np.all(np.abs(s_gpu - s_ref) <= 1e-6 * np.abs(s_ref)), (s_gpu, s_ref)
                pending[i] = s_ref
            x = out
        z = dit.drift(z)
    say(f"  skips={skips} of {T * NB}, int8 calls={checker.calls[1]}, nvfp4 calls={checker.calls[0]}, ties={ties}")
    assert skips > 0 and checker.calls[0] > 0 and checker.calls[1] > 0
    assert skips < T * NB


def test_proxy_schedule_full_size(orc):
    """42 blocks x 50 steps at 17776 tokens x 1920 hidden."""
    require_gpu()
    M, H, NB, T = 17776, 1920, 42, 50
    say(f"proxy DiT full size M={M} H={H} blocks={NB} steps={T}")
    tau, eps, dacc = _calibrate(ProxyDiT(M, H, NB, seed=10))
    say(f"  calibrated tau={tau:.4g} eps_sim={eps:.4g} delta_acc={dacc:.4g}")
    dit = ProxyDiT(M, H, NB, seed=10)
    alpha, beta = np.array([1.0, 1.0]), np.array([0.0, 0.0])
    sched = TdcScheduler(NB, M * H, alpha, beta, tau, eps, dacc)
    mirror = [orc.tdc_new() for _ in range(NB)]
    skips = 0
    routes_seen = {0: 0, 1: 0}
    deep_done = {"refresh": 0, "skip": 0}
    z = dit.x0
    for t in range(T):
        sched.begin_step()
        x = z
        for i in range(NB):
            b = sched.blocks[i]
            st = mirror[i]
            # mirror the committed state from the GPU sums (host logic parity)
            if b.state.n_refresh != st.n_refresh:
                orc.tdc_commit_refresh(st, b.sums_host.numpy().copy())
            for f in ("n_refresh", "delta_valid", "gamma_valid"):
                assert getattr(st, f) == getattr(b.state, f), (t, i, f)
            for a, c in ((st.d, b.state.d), (st.acc, b.state.acc)):
                assert a == c or (math.isnan(a) and math.isnan(c)), (t, i)
            assert np.isfinite(b.state.d) or b.state.n_refresh < 2, (t, i, b.state.d)
            skip = sched.decide(i)
            assert skip == orc.tdc_decide(st, eps, dacc), (t, i)
            if skip:
                skips += 1
                out = torch.empty_like(x)
                deep = t >= 10 and deep_done["skip"] < 3
                if deep:
                    d_before = _bits(b.delta).ravel()
                    xh = _bits(x).ravel()
                sched.skip(i, x, out)
                orc.tdc_commit_skip(st)
                if deep:
                    torch.cuda.synchronize()
                    assert np.array_equal(_bits(out).ravel(), orc.tdc_skip(xh, d_before))
                    deep_done["skip"] += 1
            else:
                _, e, r = sched.routes(i)
                sums2 = b.last_sums2 if st.gamma_valid else None
                _, _, r_o = orc.route(sums2, alpha, beta, tau)
                assert np.array_equal(r, r_o), (t, i)
                for l in range(2):
                    routes_seen[int(r[l])] += 1
                out = dit.block_forward(i, x, r)
                deep = (t >= 5 and deep_done["refresh"] < 2) or (t >= 30 and deep_done["refresh"] < 4)
                if deep:
                    torch.cuda.synchronize()
                    xh, oh = _bits(x).ravel(), _bits(out).ravel()
                    d_ref = _bits(b.delta).ravel().copy()
                    dv = bool(b.state.delta_valid)
                sched.refresh(i, x, out)
                if deep:
                    torch.cuda.synchronize()
                    s_ref = orc.tdc_refresh(xh, oh, d_ref, dv)
                    assert np.array_equal(_bits(b.delta).ravel(), d_ref)
                    s_gpu = host(b.sums)
                    assert np.all(np.abs(s_gpu - s_ref) <= 1e-6 * np.abs(s_ref)), (t, i, s_gpu, s_ref)
                    deep_done["refresh"] += 1
            x = out
        z = dit.drift(z)
    say(f"  skip rate {skips / (T * NB):.3f}, linear routes int8={routes_seen[1]} nvfp4={routes_seen[0]}, "
        f"deep checks {deep_done}")
    assert 0 < skips < T * NB
    assert routes_seen[0] > 0 and routes_seen[1] > 0
    assert deep_done["refresh"] >= 3


def test_proxy_schedule_lockstep_pdr(orc):
    require_gpu()
    M, H, NB, T = 512, 256, 6, 14
    kappa = 4.0
    say(f"proxy DiT lockstep with PDR M={M} H={H} blocks={NB} steps={T} kappa={kappa}")
    tau, eps, dacc = _calibrate(ProxyDiT(M, H, NB, seed=11))
    rho, ratios = _calibrate_pdr(ProxyDiT(M, H, NB, seed=11), kappa)
    say(f"  calibrated tau={tau:.4g} eps_sim={eps:.4g} delta_acc={dacc:.4g} rho={rho:.4g} "
        f"(ratios {min(ratios):.4g} .. {max(ratios):.4g})")
    dit = ProxyDiT(M, H, NB, seed=11)
    alpha, beta = np.array([1.0, 1.0]), np.array([0.0, 0.0])
    sched = TdcScheduler(NB, M * H, alpha, beta, tau, eps, dacc, pdr=(kappa, rho))
    mirror = [orc.tdc_new() for _ in range(NB)]
    mirror_sums2 = [None] * NB
    pending = [None] * NB
    checker = LinearChecker(orc)
    forced_n = checked_n = ties = skips = 0
    z = dit.x0
    for t in range(T):
        sched.begin_step()
        x = z
        for i in range(NB):
            if pending[i] is not None:
                orc.tdc_commit_refresh(mirror[i], pending[i])
                mirror_sums2[i] = pending[i][:2].copy()
                pending[i] = None
        for i in range(NB):
            st = mirror[i]
            skip = sched.decide(i)
            if st.n_refresh >= 2 and (_in_tie(st.d, eps) or _in_tie(st.acc + st.d, dacc)):
                ties += 1
            else:
                assert skip == orc.tdc_decide(st, eps, dacc), (t, i)
            blk = sched.blocks[i]
            xh = _bits(x)
            if skip:
                skips += 1
                out = torch.empty_like(x)
                sched.skip(i, x, out)
                orc.tdc_commit_skip(st)
            else:
                _, e, r, forced = sched.refresh_routes(i, x)
                lo, hi = orc.outlier_count_band(xh, kappa, 1e-12)
                f_lo, f_hi = orc.pdr_force(lo, xh.size, rho), orc.pdr_force(hi, xh.size, rho)
                if f_lo == f_hi:
                    assert forced == f_lo, (t, i, lo, hi, sched.last_ratio)
                else:
                    ties += 1
                checked_n += 1
                if forced:
                    forced_n += 1
                    assert np.all(r == dm.ROUTE_BF16)
                else:
                    sums2 = mirror_sums2[i] if st.gamma_valid else None
                    _, e_o, r_o = orc.route(sums2, alpha, beta, tau)
                    for l in range(2):
                        if not (sums2 is not None and _in_tie(e_o[l], tau)):
                            assert r[l] == r_o[l], (t, i, l)
                out = dit.block_forward(i, x, r, hook=checker)
                d_ref = _bits(blk.delta).ravel().copy()
                dv = bool(blk.state.delta_valid)
                sched.refresh(i, x, out)
                torch.cuda.synchronize()
                s_ref = orc.tdc_refresh(xh.ravel(), _bits(out).ravel(), d_ref, dv)
                assert np.array_equal(_bits(blk.delta).ravel(), d_ref)
                s_gpu = host(blk.sums)
                assert np.all(np.abs(s_gpu - s_ref) <= 1e-6 * np.abs(s_ref)), (s_gpu, s_ref)
                pending[i] = s_ref
            x = out
        z = dit.drift(z)
    say(f"  refresh checks={checked_n}, forced to BF16={forced_n}, skips={skips}, "
        f"linear calls bf16={checker.calls[2]} int8={checker.calls[1]} nvfp4={checker.calls[0]}, ties={ties}")
    assert 0 < forced_n < checked_n
    assert checker.calls[2] == 2 * forced_n
