"""Per-timestep driver of the Temporal Delta Cache and the DMPQ router.

Built only from libdmpq's entry points (tdc_decide / tdc_step / tdc_commit /
gate_and_route); it adds the bookkeeping of one transformer block per state
object and the single device->host boundary per timestep: the four sums a
refresh produces at step t are copied to pinned host memory asynchronously
and committed at the start of step t+1, so every routing and skip decision at
step t uses scalars of earlier steps only.

Method: 6Bit-Diffusion (gist.science summaries): TDC skips a block when its
last two residual deltas are similar and the accumulated error allows it,
reusing the cached delta, and otherwise recomputes and refreshes the cache
(§2.B); the block's Gamma from its last computed step routes its linears
(§2.A), and a block resuming after a skip has no Gamma and falls back to INT8
(§2.C).  With Purified Delta Refresh enabled (§2.C), a refresh first counts
the outliers of the block input; a ratio above rho computes every linear of
the block in BF16 for that step, overriding both the router and the INT8
fallback, so that the delta written to the cache is free of quantization
noise.  That check needs the block input of the current step, so it costs
one extra device->host copy per refreshed block.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import (OP_OUTLIER, OP_TDC, ROUTE_BF16, TDC_REFRESH, TDC_SKIP, gate_and_route,
               new_workspace, outlier_count, pdr_decide, tdc_commit, tdc_decide, tdc_init,
               tdc_step)


def spin_sync(stream=None) -> None:
    """Wait until the stream's work so far is done by polling an event.  A
    blocking synchronize sleeps until the completion interrupt wakes the
    thread, which on a busy host can leave the GPU idle for a millisecond or
    more at the one host boundary per timestep; polling reacts within
    microseconds (it keeps one core busy for the wait)."""
    ev = torch.cuda.Event()
    ev.record(stream)
    while not ev.query():
        pass


@dataclass
class BlockCache:
    state: object
    delta: torch.Tensor          # bf16 bits (int16) of the block's activation size
    sums: torch.Tensor           # device fp64[4] of the pending refresh
    sums_host: torch.Tensor      # pinned fp64[4]
    pending: bool = False        # a refresh awaits commit
    last_sums2: np.ndarray | None = None
    log: list = field(default_factory=list)


class TdcScheduler:
    def __init__(self, n_blocks: int, numel: int, alpha, beta, tau: float, eps_sim: float,
                 delta_acc: float, device="cuda", pdr=None):
        """pdr: None, or (kappa, rho) of the Purified Delta Refresh check."""
        self.alpha = np.ascontiguousarray(alpha, np.float64)
        self.beta = np.ascontiguousarray(beta, np.float64)
        self.tau, self.eps_sim, self.delta_acc = float(tau), float(eps_sim), float(delta_acc)
        self.ws = new_workspace(OP_TDC, device)
        self.pdr = None if pdr is None else (float(pdr[0]), float(pdr[1]))
        if self.pdr is not None:
            self.ws_out = new_workspace(OP_OUTLIER, device)
            self.count = torch.zeros(1, dtype=torch.float64, device=device)
            self.count_host = torch.zeros(1, dtype=torch.float64).pin_memory()
        self.last_ratio = None
        self.blocks = [BlockCache(state=tdc_init(),
                                  delta=torch.zeros(numel, dtype=torch.int16, device=device),
                                  sums=torch.zeros(4, dtype=torch.float64, device=device),
                                  sums_host=torch.zeros(4, dtype=torch.float64).pin_memory())
                       for _ in range(n_blocks)]

    def begin_step(self) -> None:
        """The one host boundary per timestep: commit last step's refreshes."""
        if not any(b.pending for b in self.blocks):
            return
        spin_sync()
        for b in self.blocks:
            if b.pending:
                s = b.sums_host.numpy().copy()
                tdc_commit(b.state, TDC_REFRESH, s)
                b.last_sums2 = s[:2].copy()
                b.pending = False

    def decide(self, i: int) -> bool:
        return tdc_decide(self.blocks[i].state, self.eps_sim, self.delta_acc)

    def routes(self, i: int):
        """Routes of block i's linears: from its Gamma, or INT8 when missing."""
        b = self.blocks[i]
        sums2 = b.last_sums2 if b.state.gamma_valid else None
        return gate_and_route(sums2, self.alpha, self.beta, self.tau)

    def refresh_routes(self, i: int, x_in: torch.Tensor):
        """Routes for a refresh of block i on input x_in [tokens x channels]:
        all BF16 when PDR is on and the outlier ratio exceeds rho, else routes(i).
        Returns (gamma, errors, routes, forced)."""
        g, e, r = self.routes(i)
        if self.pdr is None:
            return g, e, r, False
        kappa, rho = self.pdr
        outlier_count(x_in, kappa, self.count, self.ws_out)
        self.count_host.copy_(self.count)  # synchronous: the decision gates this step's linears
        n = x_in.numel()
        c = float(self.count_host[0])
        self.last_ratio = c / n if n else 0.0
        forced = pdr_decide(c, n, rho)
        if forced:
            r = np.full(len(r), ROUTE_BF16, np.uint8)
        return g, e, r, forced

    def skip(self, i: int, x_in: torch.Tensor, x_out: torch.Tensor) -> None:
        b = self.blocks[i]
        tdc_step(TDC_SKIP, x_in.view(-1), x_out.view(-1), b.delta, True)
        tdc_commit(b.state, TDC_SKIP)

    def refresh(self, i: int, x_in: torch.Tensor, x_out: torch.Tensor) -> None:
        b = self.blocks[i]
        tdc_step(TDC_REFRESH, x_in.view(-1), x_out.view(-1), b.delta,
                 bool(b.state.delta_valid), b.sums, self.ws)
        b.sums_host.copy_(b.sums, non_blocking=True)
        b.pending = True
