"""fp64 reference of the FP8 form.  TEST INFRASTRUCTURE ONLY (see package doc).

The FP8 form (TensorRT-LLM mla.py: the absorbed context path with an FP8
latent cache and the fused FP8 query, float8_e4m3fn, "the output is still in
BF16") attends over inputs given as e4m3 codes with one dequantisation scale
per tensor.  What it computes is the plain attention of the dequantised
values: this module decodes the codes exactly and hands them to
:func:`oracle.mla_ref.dense_mla`.  How the kernel rounds the softmax weights
for its FP8 P.V product is not part of the definition; the tests bound its
effect with the exact weights that :func:`attention_weights` returns.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .mla_ref import dense_mla


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 code (uint8) -> float64, exactly.

    Bit 7 is the sign, bits 6..3 the exponent field E (bias 7), bits 2..0
    the mantissa field M.  E = 0 is subnormal: (M / 8) * 2^(1 - 7).
    Otherwise (1 + M / 8) * 2^(E - 7), except that E = 15 with M = 7 is NaN;
    the format has no infinities (largest finite value 1.75 * 2^8 = 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    mag = np.where(E == 0, (M / 8.0) * 2.0 ** -6, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def dense_mla_fp8(q8: np.ndarray, kv8: np.ndarray, q_scale: float, kv_scale: float, head_dim_v: int,
                  scale: float, causal: bool = True, q_offset: int = 0, kv_offset: int = 0,
                  rows: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Shared-latent attention over FP8 inputs: q = decode(q8) * q_scale,
    kv = decode(kv8) * kv_scale (value = the first head_dim_v columns of the
    dequantised kv rows), then exactly :func:`dense_mla`."""
    q = e4m3_decode(q8) * float(q_scale)
    kv = e4m3_decode(kv8) * float(kv_scale)
    return dense_mla(q, kv, head_dim_v, scale, causal=causal, q_offset=q_offset, kv_offset=kv_offset,
                     rows=rows, heads=heads)


def attention_weights(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, q_pos: np.ndarray,
                      k_pos: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax weights of one head: (w [Nq, Nk], Z [Nq]) with w the
    normalised weights (0 for invisible keys; a row without visible keys is
    all 0) and Z = sum_j exp(s_j - max_j s_j), the row sum relative to the
    row max (1 <= Z <= number of visible keys; 0 for an empty row)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = scale * (q @ k.T)
    vis = (k_pos[None, :] <= q_pos[:, None]) if causal else np.ones(s.shape, dtype=bool)
    s = np.where(vis, s, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    Z = e.sum(axis=1)
    w = np.zeros_like(e)
    w[any_vis] = e[any_vis] / Z[any_vis, None]
    return w, Z
