"""Helpers shared by the GPU tests: moving seeded inputs to the device and
comparing device results with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

O_TOL = 1e-2     # max-abs error of bf16 outputs against the oracle
LSE_TOL = 1e-3   # max-abs error of fp32 LSE against the oracle


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bf16 GPU tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def report(name: str, got: np.ndarray, ref: np.ndarray) -> float:
    """Max-abs error with the location of the worst element; -inf must match
    -inf exactly."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    ninf_ref, ninf_got = np.isneginf(ref), np.isneginf(got)
    assert np.array_equal(ninf_ref, ninf_got), f"{name}: -inf pattern differs"
    assert not np.isnan(got).any(), f"{name}: NaN in result"
    fin = ~ninf_ref
    if not fin.any():
        return 0.0
    err = np.abs(got[fin] - ref[fin])
    i = int(np.argmax(err))
    where = np.argwhere(fin)[i]
    print(f"{name}: max abs err {err[i]:.3e} at {tuple(where)} (ref {ref[tuple(where)]:.4f})", flush=True)
    return float(err[i])
