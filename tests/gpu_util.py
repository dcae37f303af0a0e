"""Helpers shared by the GPU tests: moving seeded inputs to the device and
comparing device results with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

O_TOL = 1e-2     # max-abs error of outputs against the oracle (bf16 outputs: see bf16_bound)
LSE_TOL = 1e-3   # max-abs error of fp32 LSE against the oracle


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bf16 GPU tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bound(ref: np.ndarray) -> np.ndarray:
    """Per-element bound for a bf16 output against the exact value: the
    max-abs 1e-2 stated for this path where bf16 can meet it, one bf16 ulp
    of the exact value where it cannot.  A bf16 number has 8 significant
    bits, so the correctly rounded value alone is up to half an ulp from the
    exact one (0.0156 at |O| in [4, 8)), and a kernel result a little past
    the rounding midpoint rounds to the neighbouring value; the two bounds
    meet at |O| = 1.28."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 7)
    return np.maximum(O_TOL, ulp)


def report_o(name: str, got: np.ndarray, ref: np.ndarray) -> float:
    """bf16 output check: the largest ratio of |got - ref| to bf16_bound(ref)
    (passes at <= 1), with the max-abs error, and the max-abs error where
    |ref| < 1.28 (the bound is exactly 1e-2 there); -inf rows must match."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{name}: NaN in result"
    if got.size == 0:
        return 0.0
    err = np.abs(got - ref)
    ratio = err / bf16_bound(ref)
    i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    small = np.abs(ref) < 1.28
    print(f"{name}: max abs err {err.max():.3e}; worst against the bf16 bound {ratio[i]:.3f} at {tuple(i)} "
          f"(ref {ref[i]:.4f}, err {err[i]:.3e}); max abs err where |ref| < 1.28: "
          f"{(err[small].max() if small.any() else 0.0):.3e}", flush=True)
    return float(ratio[i])


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
