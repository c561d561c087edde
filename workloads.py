"""Seeded synthetic inputs for the dynamic mixed-precision linear layer.

Shared by the tests and the benchmark.  It holds no arithmetic of the method:
it draws numbers, scales outlier channels and rounds to bf16 with torch's own
conversion.  bf16 tensors are returned as numpy ``uint16`` bit patterns so the
CPU oracle and the GPU path consume byte-identical inputs.

Shapes follow CogVideoX-like DiT blocks (the pages evaluate CogVideoX 2B and
5B).  Token counts: 13 latent frames x 30 x 45 + 226 text tokens = 17776 for
480p-like video, 13 x 68 x 120 + 226 = 106306 for 1080p-like video.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

M_480P = 13 * 30 * 45 + 226      # 17776
M_1080P = 13 * 68 * 120 + 226    # 106306


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16) via torch's RNE conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening, via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(b).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


def n_outlier_channels(K: int) -> int:
    return 4 if K <= 256 else int(round(0.01 * K))


def activations(rng: np.random.Generator, M: int, K: int, outlier_scale: float = 50.0,
                n_out: int | None = None) -> np.ndarray:
    """N(0,1) activations [M, K] with a few whole channels scaled by 50, as bf16 bits."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    n = n_outlier_channels(K) if n_out is None else n_out
    if n:
        ch = rng.choice(K, n, replace=False)
        x[:, ch] *= np.float32(outlier_scale)
    return to_bf16_bits(x)


def weight(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """N(0, 1/K) weight [N, K] (row = output channel), as bf16 bits."""
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / math.sqrt(K))
    return to_bf16_bits(w)


def perturbed_output(rng: np.random.Generator, x_in_bits: np.ndarray,
                     gamma_target: float) -> np.ndarray:
    """X_out = X_in + c * N(0,1), with c chosen so sum|X_out-X_in| / sum|X_in| ~ gamma_target."""
    x = bf16_bits_to_f32(x_in_bits)
    c = gamma_target * float(np.mean(np.abs(x), dtype=np.float64)) / math.sqrt(2.0 / math.pi)
    noise = rng.standard_normal(x.shape, dtype=np.float32) * np.float32(c)
    return to_bf16_bits(x + noise)


def residual_block_output(rng: np.random.Generator, x_bits: np.ndarray, hidden: int) -> np.ndarray:
    """X + W2 GELU(W1 X) in fp32 on the host, rounded to bf16 (a random residual block)."""
    x = torch.from_numpy(bf16_bits_to_f32(x_bits))
    K = x.shape[1]
    w1 = torch.from_numpy(rng.standard_normal((hidden, K), dtype=np.float32)) / math.sqrt(K)
    w2 = torch.from_numpy(rng.standard_normal((K, hidden), dtype=np.float32)) / math.sqrt(hidden)
    y = x + torch.nn.functional.gelu(x @ w1.T) @ w2.T
    return to_bf16_bits(y.numpy())


@dataclass
class Linear:
    name: str
    N: int
    K: int


@dataclass
class Config:
    name: str
    M: int
    hidden: int
    linears: list = field(default_factory=list)
    seeds: tuple = ()


def linears_for(hidden: int, ffn: int) -> list:
    return [Linear("qkv", 3 * hidden, hidden), Linear("out", hidden, hidden),
            Linear("ffn_up", ffn, hidden), Linear("ffn_down", hidden, ffn)]


TINY = Config("tiny-256", 256, 256, [Linear("lin", 256, 256)], (1,))
COGVIDEOX_2B = Config("cogvideox2b-like", M_480P, 1920, linears_for(1920, 7680), (2, 3, 4, 5))
COGVIDEOX_5B = Config("cogvideox5b-like", M_480P, 3072, linears_for(3072, 12288), (6, 7, 8, 9))
PROXY_DIT = Config("proxy-dit-42x1920", M_480P, 1920, [Linear("lin1", 1920, 1920),
                                                       Linear("lin2", 1920, 1920)], (10,))
VIDEO_1080P = Config("1080p-like", M_1080P, 3072, linears_for(3072, 12288), (11, 12, 13, 14))

# Gamma targets of the four synthetic 5B-like blocks: with alpha=1, beta=0,
# tau=0.2 two blocks route to INT8 and two to NVFP4 (about 6 bits average).
GAMMA_TARGETS_5B = (0.05, 0.40, 0.05, 0.40)
ROUTER_5B = dict(alpha=1.0, beta=0.0, tau=0.2)


# ---- device-side generators (same recipes, torch's seeded GPU generator) ----
# Used where the inputs are too large to draw on the host quickly (benchmark
# steps); parity tests use the host generators above.

def device_generator(seed: int, device="cuda") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def activations_device(gen: torch.Generator, M: int, K: int, outlier_scale: float = 50.0,
                       device="cuda") -> torch.Tensor:
    """bf16 [M, K] activations: N(0,1) with round(0.01*K) channels scaled by 50."""
    x = torch.randn((M, K), generator=gen, device=device, dtype=torch.float32)
    n = n_outlier_channels(K)
    ch = torch.randperm(K, generator=gen, device=device)[:n]
    x[:, ch] *= outlier_scale
    return x.to(torch.bfloat16)


def weight_device(gen: torch.Generator, N: int, K: int, device="cuda") -> torch.Tensor:
    w = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32)
    return (w * (1.0 / math.sqrt(K))).to(torch.bfloat16)


def perturbed_output_device(gen: torch.Generator, x_in: torch.Tensor,
                            gamma_target: float) -> torch.Tensor:
    x = x_in.float()
    c = gamma_target * float(x.abs().mean(dtype=torch.float64)) / math.sqrt(2.0 / math.pi)
    noise = torch.randn(x.shape, generator=gen, device=x.device, dtype=torch.float32)
    return (x + c * noise).to(torch.bfloat16)
