"""Proxy DiT used by the schedule tests: blocks x + W2 GELU(W1 x) whose two
linears run through the library's routed quantize + GEMM entry points.

The GELU and the residual add are glue of this synthetic workload (torch,
fp32 math, bf16 storage); they are not part of the quantized-linear contract.
"""
from __future__ import annotations

import torch

import dynamic_mixed_precision_amd as dm
import workloads as wl


class ProxyLinear:
    def __init__(self, w_bf16: torch.Tensor, ws):
        N, K = w_bf16.shape
        self.N, self.K = N, K
        self.w = w_bf16.contiguous()  # the original weight, for the BF16 (PDR) route
        self.cw = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
        self.sw = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
        self.gw = torch.zeros(1, device="cuda")
        self.qw = torch.empty((N, K), dtype=torch.int8, device="cuda")
        self.swr = torch.empty(N, device="cuda")
        dm.prep_weight(w_bf16, self.cw, self.sw, self.gw, self.qw, self.swr, ws)


class QuantBuffers:
    def __init__(self, M: int, K: int):
        self.q = torch.empty((M, K), dtype=torch.int8, device="cuda")
        self.s = torch.empty(M, device="cuda")
        self.c = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
        self.sc = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
        self.g = torch.zeros(1, device="cuda")


def routed_linear(x: torch.Tensor, lin: ProxyLinear, route: int, qb: QuantBuffers, ws,
                  hook=None) -> torch.Tensor:
    """Hadamard + quant at the routed precision, then the quantized GEMM (bf16 out);
    the BF16 route is the unquantized GEMM on the original weight."""
    M = x.shape[0]
    y = torch.empty((M, lin.N), dtype=torch.bfloat16, device="cuda")
    if route == dm.ROUTE_BF16:
        dm.gemm_bf16(x.view(torch.int16), lin.w.view(torch.int16), y, dm.OUT_BF16)
    elif route == dm.ROUTE_INT8:
        dm.hadamard_quant_int8(x, qb.q, qb.s)
        dm.qgemm_int8(qb.q, qb.s, lin.qw, lin.swr, y, dm.OUT_BF16)
    else:
        dm.hadamard_quant_nvfp4(x, qb.c, qb.sc, qb.g, ws)
        dm.qgemm_nvfp4(qb.c, qb.sc, qb.g, lin.cw, lin.sw, lin.gw, y, dm.OUT_BF16)
    if hook is not None:
        hook(x, lin, route, qb, y)
    return y


RESIDUAL_W2_SCALE = 0.3


class ProxyDiT:
    """n_blocks residual blocks, hidden H -> H -> H.  W1 ~ N(0, 1/H); W2 ~
    N(0, (0.3)^2 / H), so each block adds a modest residual (Gamma of order
    0.1-0.5) and 42 blocks without normalization stay well inside bf16 range.
    Each timestep feeds the blocks a latent z_t = z_{t-1} + 0.02 N(0, 1)."""

    def __init__(self, M: int, H: int, n_blocks: int, seed: int):
        self.M, self.H = M, H
        gen = wl.device_generator(seed)
        self.ws = dm.new_workspace(dm.OP_PREP_WEIGHT)
        self.blocks = []
        for _ in range(n_blocks):
            w1 = wl.weight_device(gen, H, H)
            w2 = (wl.weight_device(gen, H, H).float() * RESIDUAL_W2_SCALE).to(torch.bfloat16)
            self.blocks.append((ProxyLinear(w1, self.ws), ProxyLinear(w2, self.ws)))
        self.qb = QuantBuffers(M, H)
        self.x0 = wl.activations_device(gen, M, H)
        self.gen = gen

    def drift(self, x: torch.Tensor) -> torch.Tensor:
        """x_t = x_{t-1} + 0.02 * N(0, 1) (smoothly drifting inputs)."""
        n = torch.randn(x.shape, generator=self.gen, device="cuda", dtype=torch.float32)
        return (x.float() + 0.02 * n).to(torch.bfloat16)

    def block_forward(self, i: int, x: torch.Tensor, routes, hook=None) -> torch.Tensor:
        lin1, lin2 = self.blocks[i]
        h = routed_linear(x, lin1, int(routes[0]), self.qb, self.ws, hook)
        h = torch.nn.functional.gelu(h.float()).to(torch.bfloat16)
        y = routed_linear(h, lin2, int(routes[1]), self.qb, self.ws, hook)
        return (x.float() + y.float()).to(torch.bfloat16)
