"""Helpers for the GPU parity tests: byte-exact numpy <-> device copies."""
import numpy as np
import pytest
import torch

import dynamic_mixed_precision_amd as dm

_VIEW = {np.dtype(np.uint16): torch.int16, np.dtype(np.uint8): torch.uint8,
         np.dtype(np.int8): torch.int8, np.dtype(np.float32): torch.float32,
         np.dtype(np.float64): torch.float64, np.dtype(np.int32): torch.int32}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dm.lib()  # fails loudly if the HIP library is not built


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def empty(shape, dtype) -> torch.Tensor:
    return torch.empty(shape, dtype=_VIEW[np.dtype(dtype)], device="cuda")


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def say(msg: str) -> None:
    print(msg, flush=True)
