"""Helpers shared by the GPU tests: moving seeded inputs to the device and
comparing device results with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

O_TOL = 1e-2     # max-abs error of outputs against the oracle (bf16 outputs: see bf16_bound)
LSE_TOL = 1e-3   # max-abs error of fp32 LSE against the oracle
BF16_WIDE = 2.0  # |O| from which a bf16 output is held to "the rounding of a value within 1e-2"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> bf16 GPU tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bound(ref: np.ndarray) -> np.ndarray:
    """Per-element bound for a bf16 output against the exact value.

    The kernels compute in fp32 and round once to bf16 (round to nearest
    even).  Below |O| = 2 the bound is the flat max-abs 1e-2 stated for this
    path.  From |O| = 2 on it is half an ulp of the exact value plus 1e-2:
    the bf16 output must be the rounding of a value within 1e-2 of the exact
    one.  Half an ulp is 2^-8 on [2, 4) and 2^-7 on [4, 8), so the rounding
    alone takes most (or more than all) of a flat 1e-2 there, while the fp32
    value before it carries the error of the bf16 P in the P.V product (up to
    about 5e-3 measured).  The fp32-output twins of the tests hold that fp32
    value to 1e-2 everywhere and check that the bf16 result is its
    round-to-nearest-even bit for bit."""
    a = np.abs(np.asarray(ref, dtype=np.float64))
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 8)
    return np.where(a < BF16_WIDE, O_TOL, half_ulp + O_TOL)


def report_o(name: str, got: np.ndarray, ref: np.ndarray) -> float:
    """bf16 output check: the largest ratio of |got - ref| to bf16_bound(ref)
    (passes at <= 1), with the max-abs error overall and where |ref| < 2 (the
    bound is exactly 1e-2 there)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{name}: NaN in result"
    if got.size == 0:
        return 0.0
    err = np.abs(got - ref)
    ratio = err / bf16_bound(ref)
    i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    small = np.abs(ref) < BF16_WIDE
    print(f"{name}: max abs err {err.max():.3e}; worst against the bf16 bound {ratio[i]:.3f} at {tuple(i)} "
          f"(ref {ref[i]:.4f}, err {err[i]:.3e}); max abs err where |ref| < {BF16_WIDE:g}: "
          f"{(err[small].max() if small.any() else 0.0):.3e}; largest |ref| {np.abs(ref).max():.3f}", flush=True)
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


def assert_rne_of(name: str, bf16_out: torch.Tensor, f32_out: torch.Tensor) -> None:
    """The bf16 result is bit for bit the round-to-nearest-even of the fp32
    result of the same call (torch's float32 -> bfloat16 conversion rounds
    to nearest even): the only difference between the two output types is
    that one rounding."""
    assert bf16_out.dtype == torch.bfloat16 and f32_out.dtype == torch.float32
    assert bf16_out.shape == f32_out.shape, (name, bf16_out.shape, f32_out.shape)
    want = f32_out.to(torch.bfloat16)
    same = bf16_out.view(torch.int16) == want.view(torch.int16)
    n_bad = int((~same).sum())
    print(f"{name}: bf16 = RNE(fp32) on {same.numel() - n_bad} of {same.numel()} elements", flush=True)
    assert n_bad == 0, f"{name}: {n_bad} bf16 outputs are not the rounding of the fp32 output"
