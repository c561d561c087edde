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
(§2.C).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import (OP_TDC, TDC_REFRESH, TDC_SKIP, gate_and_route, new_workspace, tdc_commit,
               tdc_decide, tdc_init, tdc_step)


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
                 delta_acc: float, device="cuda"):
        self.alpha = np.ascontiguousarray(alpha, np.float64)
        self.beta = np.ascontiguousarray(beta, np.float64)
        self.tau, self.eps_sim, self.delta_acc = float(tau), float(eps_sim), float(delta_acc)
        self.ws = new_workspace(OP_TDC, device)
        self.blocks = [BlockCache(state=tdc_init(),
                                  delta=torch.zeros(numel, dtype=torch.int16, device=device),
                                  sums=torch.zeros(4, dtype=torch.float64, device=device),
                                  sums_host=torch.zeros(4, dtype=torch.float64).pin_memory())
                       for _ in range(n_blocks)]

    def begin_step(self) -> None:
        """The one host boundary per timestep: commit last step's refreshes."""
        if not any(b.pending for b in self.blocks):
            return
        torch.cuda.current_stream().synchronize()
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
