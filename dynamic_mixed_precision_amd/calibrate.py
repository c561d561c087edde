"""Offline fit of the DMPQ router's linear error model E_l = alpha_l * Gamma + beta_l.

Method: 6Bit-Diffusion predicts each linear's quantization error from the
block's Gamma of the previous step with a pre-fitted linear model and routes
the linear to INT8 when the prediction exceeds tau (gist.science summaries,
§2.A "Mechanism" items 2-3).  The pages do not say which error the model
predicts; here it is the relative L1 error of the linear's NVFP4 output
against its full-precision (BF16) output, the same L1 measure as Gamma:

    E_l = sum |Y_nvfp4 - Y_bf16| / sum |Y_bf16|.

Every number comes from the library's kernels: the NVFP4 route
(hadamard_quant_nvfp4 + qgemm_nvfp4), the BF16 GEMM, and gamma_sums, whose
two sums on (Y_bf16, Y_nvfp4) are exactly the numerator and denominator
above.  The fit itself is ordinary least squares on the host.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (OP_GAMMA, OP_QUANT_NVFP4, OUT_BF16, gamma_sums, gemm_bf16, hadamard_quant_nvfp4,
               new_workspace, qgemm_nvfp4)


class ErrorProbe:
    """Relative L1 error of the NVFP4 route of one linear, measured on the GPU."""

    def __init__(self, M: int, K: int, N: int, device="cuda"):
        self.codes = torch.empty((M, K // 2), dtype=torch.uint8, device=device)
        self.scales = torch.empty((M, K // 16), dtype=torch.uint8, device=device)
        self.g = torch.zeros(1, device=device)
        self.y_q = torch.empty((M, N), dtype=torch.int16, device=device)
        self.y_ref = torch.empty((M, N), dtype=torch.int16, device=device)
        self.sums = torch.zeros(2, dtype=torch.float64, device=device)
        self.ws_q = new_workspace(OP_QUANT_NVFP4, device)
        self.ws_g = new_workspace(OP_GAMMA, device)

    def __call__(self, x, w_bf16, cw, sw, gw) -> float:
        """x [M x K] and w_bf16 [N x K] bf16 (int16 bits or bfloat16); (cw, sw, gw)
        the linear's NVFP4 weight.  Returns E_l (synchronizes)."""
        x16 = x.view(torch.int16)
        hadamard_quant_nvfp4(x16, self.codes, self.scales, self.g, self.ws_q)
        qgemm_nvfp4(self.codes, self.scales, self.g, cw, sw, gw, self.y_q, OUT_BF16)
        gemm_bf16(x16, w_bf16.view(torch.int16), self.y_ref, OUT_BF16)
        gamma_sums(self.y_ref.view(-1), self.y_q.view(-1), self.sums, self.ws_g)
        s1, s2 = self.sums.tolist()
        return s1 / s2 if s2 > 0 else (0.0 if s1 == 0 else float("inf"))


def fit_router(gammas, errors):
    """Least-squares alpha, beta with errors ~ alpha * gammas + beta.

    gammas, errors: [n_samples] (one linear) or [n_samples, n_linears]
    (gammas may then be [n_samples], shared by the block's linears).
    Returns (alpha, beta) as arrays over linears and the RMS residual."""
    e = np.asarray(errors, np.float64)
    if e.ndim == 1:
        e = e[:, None]
    g = np.asarray(gammas, np.float64)
    if g.ndim == 1:
        g = np.repeat(g[:, None], e.shape[1], axis=1)
    if g.shape != e.shape or e.shape[0] < 2:
        raise ValueError("need matching samples, at least two")
    alpha = np.empty(e.shape[1])
    beta = np.empty(e.shape[1])
    rms = np.empty(e.shape[1])
    for l in range(e.shape[1]):
        A = np.stack([g[:, l], np.ones(len(g))], axis=1)
        (a, b), *_ = np.linalg.lstsq(A, e[:, l], rcond=None)
        alpha[l], beta[l] = a, b
        rms[l] = float(np.sqrt(np.mean((A @ np.array([a, b]) - e[:, l]) ** 2)))
    return alpha, beta, rms
