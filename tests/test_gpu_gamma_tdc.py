"""GPU parity: Gamma sums, TDC skip and refresh against the oracle.

Sums within 1e-6 relative (the kernels add 8 fp32 terms per lane before
going to fp64, a relative error below 4.2e-7 for non-negative terms), skip
output and cached delta bit-exact, decisions identical, and the sums
bit-identical from run to run.
"""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm
import workloads
from gpu_util import dev, empty, host, require_gpu, say

pytestmark = pytest.mark.gpu

REL = 1e-6
SIZES = [1, 7, 8, 1000, 256 * 256, 17776 * 1920 // 8 + 3, 17776 * 3072]


def _close(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.all(np.abs(a - b) <= REL * np.abs(b))


def _gpu_gamma(xi, xo):
    s = torch.zeros(2, dtype=torch.float64, device="cuda")
    ws = dm.new_workspace(dm.OP_GAMMA)
    dm.gamma_sums(dev(xi), dev(xo), s, ws)
    torch.cuda.synchronize()
    return host(s)


@pytest.mark.parametrize("n", SIZES)
def test_gamma_sums_parity(orc, n):
    require_gpu()
    say(f"gamma_sums n={n}")
    rng = np.random.default_rng(n)
    xi = workloads.activations(rng, 1, n, n_out=0).ravel()
    xo = workloads.perturbed_output(rng, xi.reshape(1, -1), 0.3).ravel()
    s0 = orc.gamma_sums(xi, xo)
    s1 = _gpu_gamma(xi, xo)
    assert _close(s1, s0), (s1, s0)
    s2 = _gpu_gamma(xi, xo)
    assert np.array_equal(s1, s2)  # deterministic


def test_gamma_closed_forms_gpu():
    require_gpu()
    say("gamma closed forms")
    x = workloads.activations(np.random.default_rng(80), 64, 256)
    xf = workloads.bf16_bits_to_f32(x)
    s = _gpu_gamma(x, x)
    assert s[0] == 0.0 and s[1] > 0
    s = _gpu_gamma(x, workloads.to_bf16_bits(-xf))
    assert s[0] == 2 * s[1]
    z = np.zeros_like(x)
    assert np.array_equal(_gpu_gamma(z, z), [0.0, 0.0])
    s = _gpu_gamma(np.zeros(0, np.uint16), np.zeros(0, np.uint16))
    assert np.array_equal(s, [0.0, 0.0])


@pytest.mark.parametrize("n", SIZES)
def test_tdc_skip_parity(orc, n):
    require_gpu()
    say(f"tdc_step SKIP n={n}")
    rng = np.random.default_rng(n + 1)
    xi = workloads.activations(rng, 1, n, n_out=0).ravel()
    d = workloads.to_bf16_bits(0.1 * rng.standard_normal(n).astype(np.float32))
    out = empty((n,), np.uint16)
    dm.tdc_step(dm.TDC_SKIP, dev(xi), out, dev(d), True)
    torch.cuda.synchronize()
    assert np.array_equal(host(out, np.uint16), orc.tdc_skip(xi, d))


@pytest.mark.parametrize("dv", [False, True])
@pytest.mark.parametrize("n", SIZES)
def test_tdc_refresh_parity(orc, n, dv):
    require_gpu()
    say(f"tdc_step REFRESH n={n} delta_valid={dv}")
    rng = np.random.default_rng(n + 2)
    xi = workloads.activations(rng, 1, n, n_out=0).ravel()
    xo = workloads.perturbed_output(rng, xi.reshape(1, -1), 0.2).ravel()
    d_prev = workloads.to_bf16_bits(0.25 * rng.standard_normal(n).astype(np.float32))
    d_ref = d_prev.copy()
    s0 = orc.tdc_refresh(xi, xo, d_ref, dv)
    dg = dev(d_prev)
    s = torch.zeros(4, dtype=torch.float64, device="cuda")
    dm.tdc_step(dm.TDC_REFRESH, dev(xi), dev(xo), dg, dv, s, dm.new_workspace(dm.OP_TDC))
    torch.cuda.synchronize()
    assert np.array_equal(host(dg, np.uint16), d_ref)
    s1 = host(s)
    assert _close(s1, s0), (s1, s0)
    if not dv:
        assert s1[2] == 0 and s1[3] == 0


def test_tdc_gamma_1080p_size(orc):
    """The 1080p-like block input (106306 tokens x 3072 = 327 M elements), the
    largest configuration: Gamma sums, a refresh with a valid delta, and a skip
    at full size.  The inputs tile a seeded 8 M-element draw (the same value
    distribution, at the full size's grid and partial-sum layout; drawing 327 M
    values takes minutes).  The refresh's delta is compared whole, the skip
    output, which is elementwise, on a sample of positions."""
    require_gpu()
    n = workloads.M_1080P * 3072
    say(f"gamma + tdc at the 1080p size n={n}")
    rng = np.random.default_rng(1080)
    b = 1 << 23
    xi0 = workloads.activations(rng, 1, b, n_out=0).ravel()
    xo0 = workloads.perturbed_output(rng, xi0.reshape(1, -1), 0.2).ravel()
    d0 = workloads.to_bf16_bits(0.25 * rng.standard_normal(b).astype(np.float32))
    reps = -(-n // b)
    xi, xo, d_prev = (np.tile(a, reps)[:n] for a in (xi0, xo0, d0))
    assert _close(_gpu_gamma(xi, xo), orc.gamma_sums(xi, xo))
    d_ref = d_prev.copy()
    s0 = orc.tdc_refresh(xi, xo, d_ref, True)
    xig, dg = dev(xi), dev(d_prev)
    s = torch.zeros(4, dtype=torch.float64, device="cuda")
    dm.tdc_step(dm.TDC_REFRESH, xig, dev(xo), dg, True, s, dm.new_workspace(dm.OP_TDC))
    torch.cuda.synchronize()
    assert np.array_equal(host(dg, np.uint16), d_ref)
    assert _close(host(s), s0), (host(s), s0)
    out = empty((n,), np.uint16)
    dm.tdc_step(dm.TDC_SKIP, xig, out, dg, True)
    torch.cuda.synchronize()
    idx = np.unique(np.concatenate([rng.integers(0, n, 1 << 20), np.arange(n - 64, n)]))
    got = host(out, np.uint16)[idx]
    assert np.array_equal(got, orc.tdc_skip(xi[idx], d_ref[idx]))


def test_tdc_schedule_lockstep(orc):
    """A short TDC schedule where the GPU computes every device step and the
    oracle recomputes each one from the GPU's own inputs; decisions come from
    the library's host functions and the oracle's, and must agree."""
    require_gpu()
    say("tdc lockstep schedule")
    rng = np.random.default_rng(81)
    M, H = 256, 256
    x = workloads.activations(rng, M, H)
    c = workloads.to_bf16_bits(0.5 * rng.standard_normal((M, H)).astype(np.float32))
    eps, dacc = 0.05, 0.08
    st_l, st_o = dm.tdc_init(), orc.tdc_new()
    delta = torch.zeros(M * H, dtype=torch.int16, device="cuda")
    ws = dm.new_workspace(dm.OP_TDC)
    sums = torch.zeros(4, dtype=torch.float64, device="cuda")
    pattern = []
    for t in range(24):
        skip_l = dm.tdc_decide(st_l, eps, dacc)
        skip_o = orc.tdc_decide(st_o, eps, dacc)
        assert skip_l == skip_o, t
        xi = dev(x).view(-1)
        if skip_l:
            out = torch.empty_like(xi)
            d_before = host(delta, np.uint16).copy()
            dm.tdc_step(dm.TDC_SKIP, xi, out, delta, True)
            torch.cuda.synchronize()
            assert np.array_equal(host(out, np.uint16), orc.tdc_skip(x.ravel(), d_before))
            dm.tdc_commit(st_l, dm.TDC_SKIP)
            orc.tdc_commit_skip(st_o)
        else:
            # the "block": out = in * (1 + small drift) + c, computed on the host
            f = workloads.bf16_bits_to_f32(x)
            xo = workloads.to_bf16_bits(f * np.float32(1.0 + 0.002 * t) +
                                        workloads.bf16_bits_to_f32(c))
            d_ref = host(delta, np.uint16).copy()
            s0 = orc.tdc_refresh(x.ravel(), xo.ravel(), d_ref, bool(st_o.delta_valid))
            dm.tdc_step(dm.TDC_REFRESH, xi, dev(xo).view(-1), delta, bool(st_l.delta_valid),
                        sums, ws)
            torch.cuda.synchronize()
            s1 = host(sums)
            assert np.array_equal(host(delta, np.uint16), d_ref)
            assert _close(s1, s0)
            dm.tdc_commit(st_l, dm.TDC_REFRESH, s1)
            orc.tdc_commit_refresh(st_o, s0)
        pattern.append(int(skip_l))
        x = workloads.to_bf16_bits(workloads.bf16_bits_to_f32(x) + np.float32(0.01) *
                                   rng.standard_normal((M, H)).astype(np.float32))
    assert 0 < sum(pattern) < len(pattern), pattern


@pytest.mark.parametrize("n", [1000, 17776 * 3072])
def test_refresh_sums_are_gamma_sums(orc, n):
    """A REFRESH returns S1 = sum |out - in| and S2 = sum |in| over the same
    tensors as dmpq_gamma_sums, so the next step's router can take Gamma from
    it (the bench's default).  The two kernels add in different orders: each
    is within 1e-6 of the oracle, so within 2e-6 of each other, and the oracle
    itself defines both sums alike."""
    require_gpu()
    say(f"refresh sums vs gamma sums n={n}")
    rng = np.random.default_rng(n + 5)
    xi = workloads.activations(rng, 1, n, n_out=0).ravel()
    xo = workloads.perturbed_output(rng, xi.reshape(1, -1), 0.2).ravel()
    g = _gpu_gamma(xi, xo)
    s = torch.zeros(4, dtype=torch.float64, device="cuda")
    dm.tdc_step(dm.TDC_REFRESH, dev(xi), dev(xo), dev(np.zeros(n, np.uint16)), False, s,
                dm.new_workspace(dm.OP_TDC))
    torch.cuda.synchronize()
    r = host(s)[:2]
    assert np.all(np.abs(r - g) <= 2 * REL * np.abs(g)), (r, g)
    d_ref = np.zeros(n, np.uint16)
    assert np.array_equal(orc.tdc_refresh(xi, xo, d_ref, False)[:2], orc.gamma_sums(xi, xo))
    alpha, beta = np.ones(4), np.zeros(4)
    gamma = g[0] / g[1]
    for tau in (0.5 * gamma, 2.0 * gamma):
        assert np.array_equal(dm.gate_and_route(g, alpha, beta, tau)[2],
                              dm.gate_and_route(r, alpha, beta, tau)[2])
