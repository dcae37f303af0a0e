"""Seeded synthetic inputs for shared-latent MLA attention.

This module only draws random numbers and stores them as bfloat16 bit
patterns.  It holds none of the attention arithmetic, so both the fp64 oracle
(used by the tests) and the HIP path can be fed from it without sharing any of
the method's code.

Every tensor is drawn with ``numpy.random.default_rng(seed)`` as float32
``standard_normal`` and rounded to bfloat16 round-to-nearest-even, in the order
the workload lists its tensors.  The shapes follow the pages:

* shared-latent rows of 512 latent + 64 RoPE columns with one KV head and
  ``head_dim_v`` = 512 read from the KV prefix (TT-NN ``ring_mla``,
  "Parameters" and ``head_dim_v``; TensorRT-LLM ``mla.py``, ``MLA.__init__``
  building the absorbed ``mqa`` backend with ``num_kv_heads=1``);
* the split query/key ring step with nope 128 + RoPE 64 and V 128, ``seqLen``
  per sequence and ``prevOut``/``prevLse`` (Ascend ``RingMLAOperation``,
  member table of ``AtbRingMLAGetWorkspaceSize``);
* the sparse top-k latent path with ``q_lift``, ``q_pe``, ``c_kv``, ``k_pe``
  and flat int32 indices (NKI ``mla_sparse_attention_cte_kernel``,
  "Parameters");
* the V-up projection after latent attention, with a synthetic weight
  ``w_uv`` [H, 128, 512] (TensorRT-LLM ``mla.py``, ``v_b_proj``): there are no
  trained weights here, so it is drawn N(0,1) and divided by sqrt(512) before
  the bf16 rounding, which keeps the projected values at the scale of the
  latent output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

SCALE_192 = 1.0 / math.sqrt(192.0)   # 1/sqrt(qk_nope 128 + qk_rope 64)


# ---------------------------------------------------------------------------
# bfloat16 storage helpers (bit manipulation only)
# ---------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern (uint16), round to nearest even.

    Inputs are finite draws from a normal distribution, so no NaN handling is
    needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 26) -> np.ndarray:
    """Draw N(0,1) float32 and round to bf16 bits, in bounded chunks so that a
    1.2 GB tensor does not need 3x its size of temporaries."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------
@dataclass
class DenseCase:
    """Shared-latent causal attention: q [B,H,N,dk], kv [B,1,Nkv,dk] (bf16 bits)."""
    q: np.ndarray
    kv: np.ndarray
    head_dim_v: int
    scale: float
    causal: bool = True
    q_offset: int = 0
    kv_offset: int = 0
    n_chunks: int = 1      # >1: processed as a one-GPU ring of contiguous chunks
    name: str = ""


@dataclass
class SplitCase:
    """Split query/key ring step with per-sequence lengths, [T, H, D] layouts."""
    seq_lens: np.ndarray   # int32 [n_seqs], or [2, n_seqs]: query lengths, then key lengths
    q1: np.ndarray         # [T, H, 128]
    q2: np.ndarray         # [T, H, 64]
    k1: np.ndarray         # [Tk, Hkv, 128] (Tk = T unless key lengths are given)
    k2: np.ndarray         # [Tk, Hkv, 64]
    v: np.ndarray          # [Tk, Hkv, 128]
    prev_out: Optional[np.ndarray]   # [T, H, 128] bf16 bits
    prev_lse: Optional[np.ndarray]   # [H, T] float32
    scale: float
    causal: bool = True
    name: str = ""


@dataclass
class SparseCase:
    """Top-k sparse latent attention, B = 1."""
    q_lift: np.ndarray     # [B, S, H, L]
    q_pe: np.ndarray       # [B, S, H, R]
    c_kv: np.ndarray       # [B, S_kv, L]
    k_pe: np.ndarray       # [B, S_kv, R]
    idx: np.ndarray        # int32 [B, S, K]
    positions: np.ndarray  # int64 [S], query positions (the causal range of the draw)
    scale: float
    name: str = ""


@dataclass
class DecodeCase:
    """Token generation: the newest query of each sequence over its cache rows."""
    q: np.ndarray          # [B, H, 576] (one query per sequence)
    kv: np.ndarray         # [B, Nkv, 576] latent cache rows (512 latent + 64 RoPE)
    kv_lens: np.ndarray    # int32 [B] valid rows per sequence
    head_dim_v: int
    scale: float
    name: str = ""


def dense_case(B: int = 1, H: int = 4, N: int = 128, Nkv: Optional[int] = None,
               dk: int = 576, dv: int = 512, seed: int = 0, scale: float = SCALE_192,
               causal: bool = True, q_offset: int = 0, kv_offset: int = 0,
               n_chunks: int = 1, name: str = "") -> DenseCase:
    rng = np.random.default_rng(seed)
    Nkv = N if Nkv is None else Nkv
    q = normal_bf16(rng, (B, H, N, dk))
    kv = normal_bf16(rng, (B, 1, Nkv, dk))
    return DenseCase(q, kv, dv, scale, causal, q_offset, kv_offset, n_chunks, name)


def split_case(seq_lens: Optional[List[int]] = None, n_seqs: int = 8, len_lo: int = 1024,
               len_hi: int = 8192, H: int = 32, Hkv: int = 32, d_nope: int = 128,
               d_rope: int = 64, dv: int = 128, seed: int = 0, scale: float = SCALE_192,
               causal: bool = True, with_prev: bool = True, lse_hi: float = 12.0,
               name: str = "", kv_lens: Optional[List[int]] = None) -> SplitCase:
    """With ``kv_lens`` the key tensors hold their own per-sequence lengths
    (seq_lens becomes [2, n_seqs]: query lengths, then key lengths)."""
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        lens = rng.integers(len_lo, len_hi, n_seqs, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(seq_lens, dtype=np.int32)
    T = int(lens.sum())
    Tk = T if kv_lens is None else int(np.sum(kv_lens))
    q1 = normal_bf16(rng, (T, H, d_nope))
    q2 = normal_bf16(rng, (T, H, d_rope))
    k1 = normal_bf16(rng, (Tk, Hkv, d_nope))
    k2 = normal_bf16(rng, (Tk, Hkv, d_rope))
    v = normal_bf16(rng, (Tk, Hkv, dv))
    if kv_lens is not None:
        if len(kv_lens) != len(lens):
            raise ValueError("one key length per sequence")
        lens = np.stack([lens, np.asarray(kv_lens, dtype=np.int32)])
    prev_out = prev_lse = None
    if with_prev:
        prev_out = normal_bf16(rng, (T, H, dv))
        prev_lse = rng.uniform(0.0, lse_hi, (H, T)).astype(np.float32)
    return SplitCase(lens, q1, q2, k1, k2, v, prev_out, prev_lse, scale, causal, name)


def sparse_case(S: int = 4096, S_kv: int = 16384, pos0: int = 12288, H: int = 128,
                L: int = 512, R: int = 64, K: int = 2048, seed: int = 0,
                scale: float = SCALE_192, name: str = "") -> SparseCase:
    """Per query i at position pos0 + i, K distinct indices drawn uniformly from
    the causal range [0, pos], kept in drawn order."""
    if pos0 + 1 < K:
        raise ValueError("the first query must have at least K visible rows")
    rng = np.random.default_rng(seed)
    q_lift = normal_bf16(rng, (1, S, H, L))
    q_pe = normal_bf16(rng, (1, S, H, R))
    c_kv = normal_bf16(rng, (1, S_kv, L))
    k_pe = normal_bf16(rng, (1, S_kv, R))
    pos = np.arange(pos0, pos0 + S, dtype=np.int64)
    if pos[-1] >= S_kv:
        raise ValueError("query positions must lie inside the cache")
    idx = np.empty((1, S, K), dtype=np.int32)
    for i in range(S):
        idx[0, i] = rng.choice(int(pos[i]) + 1, K, replace=False)
    return SparseCase(q_lift, q_pe, c_kv, k_pe, idx, pos, scale, name)


def decode_case(B: int = 64, H: int = 128, Nkv: int = 8192, kv_lens: Optional[List[int]] = None,
                len_lo: Optional[int] = None, dk: int = 576, dv: int = 512, seed: int = 0,
                scale: float = SCALE_192, name: str = "") -> DecodeCase:
    """q then kv drawn N(0,1) -> bf16; valid lengths as given, else drawn
    uniformly in [len_lo, Nkv] (after the tensors) when len_lo is set, else
    Nkv for every sequence."""
    rng = np.random.default_rng(seed)
    q = normal_bf16(rng, (B, H, dk))
    kv = normal_bf16(rng, (B, Nkv, dk))
    if kv_lens is not None:
        lens = np.asarray(kv_lens, dtype=np.int32)
    elif len_lo is not None:
        lens = rng.integers(len_lo, Nkv, B, endpoint=True).astype(np.int32)
    else:
        lens = np.full(B, Nkv, dtype=np.int32)
    return DecodeCase(q, kv, lens, dv, scale, name)


# The five workloads the method is measured and checked on (and decode,
# the next step beside them).
def tiny(seed: int = 0) -> DenseCase:
    return dense_case(B=1, H=4, N=128, seed=seed, name="tiny causal MLA H=4 N=128")


def ring4(seed: int = 0) -> DenseCase:
    return dense_case(B=1, H=16, N=4096, seed=seed, n_chunks=4,
                      name="ring causal MLA H=16 N=4096 in 4 chunks of 1024")


def dsv3_prefill(seed: int = 0) -> DenseCase:
    return dense_case(B=1, H=128, N=8192, seed=seed,
                      name="DeepSeek-V3 absorbed MLA prefill H=128 N=8192")


def split_ring_step(seed: int = 0) -> SplitCase:
    return split_case(seed=seed, name="split q/k varlen ring step 8 seqs H=32")


def sparse_topk(seed: int = 0) -> SparseCase:
    return sparse_case(seed=seed, name="sparse top-k MLA S=4096 S_kv=16384 H=128 K=2048")


@dataclass
class VupCase:
    o: np.ndarray      # [B, H, T, L] latent attention output (bf16 bits)
    w_uv: np.ndarray   # [H, dvh, L] (bf16 bits)
    name: str = ""


def vup_case(B: int = 1, H: int = 4, T: int = 64, L: int = 512, dvh: int = 128, seed: int = 0,
             name: str = "") -> VupCase:
    rng = np.random.default_rng(seed)
    o = normal_bf16(rng, (B, H, T, L))
    w = to_bf16_bits(rng.standard_normal((H, dvh, L), dtype=np.float32) / np.float32(math.sqrt(L)))
    return VupCase(o, w, name)


def dsv3_vup(seed: int = 0) -> VupCase:
    return vup_case(B=1, H=128, T=8192, seed=seed, name="DeepSeek-V3 V-up projection H=128 T=8192")


def dsv3_decode(seed: int = 0) -> DecodeCase:
    return decode_case(B=64, H=128, Nkv=8192, seed=seed,
                       name="DeepSeek-V3 absorbed MLA decode B=64 H=128 KV=8192")


# ---------------------------------------------------------------------------
# FP8 inputs (TensorRT-LLM mla.py, forward_absorption_context: the fused FP8
# query [tokens, heads, kv_lora_rank + qk_rope_head_dim] in float8_e4m3fn
# written at unit scale, and the FP8 latent cache with its dequantisation
# scale).  The codes are the OCP FP8 E4M3 format ("e4m3fn": 1 sign bit, 4
# exponent bits of bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN,
# largest finite value 448).  Quantising a draw to a code is input
# preparation, like the bf16 rounding above; no attention arithmetic.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn code (uint8), round to nearest even, saturating at
    +-448 (the draws are finite).  On the float32 bit patterns: in the normal
    range the 20 mantissa bits e4m3 drops are rounded off and the exponent
    is rebiased from 127 to 7; below 2^-6 the value is a multiple of 2^-9."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    sign = ((u >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8)
    a = u & np.uint32(0x7FFFFFFF)
    r = (a + np.uint32(0x7FFFF) + ((a >> np.uint32(20)) & np.uint32(1))) >> np.uint32(20)
    code = np.minimum(r.astype(np.int64) - ((127 - 7) << 3), 0x7E)          # 0x7E = 448
    small = a < np.uint32(0x3C800000)                                         # |x| < 2^-6
    code[small] = np.rint(a[small].view(np.float32) * np.float32(512.0)).astype(np.int64)
    return code.astype(np.uint8) | sign


def normal_e4m3(rng: np.random.Generator, shape, std: float = 1.0, chunk: int = 1 << 26) -> np.ndarray:
    """Draw N(0, std^2) float32 and store it as e4m3 codes at unit scale, in
    bounded chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = to_e4m3_codes(rng.standard_normal(e - s, dtype=np.float32) * np.float32(std))
    return out.reshape(shape)


@dataclass
class Fp8DenseCase:
    """Shared-latent causal attention over FP8 inputs: q8 [B,H,N,576] and kv8
    [B,1,Nkv,576] e4m3 codes, dequantised as code * q_scale and
    code * kv_scale."""
    q8: np.ndarray
    kv8: np.ndarray
    q_scale: float
    kv_scale: float
    head_dim_v: int
    scale: float
    causal: bool = True
    q_offset: int = 0
    kv_offset: int = 0
    name: str = ""


def fp8_dense_case(B: int = 1, H: int = 4, N: int = 128, Nkv: Optional[int] = None, dk: int = 576,
                   dv: int = 512, seed: int = 0, scale: float = SCALE_192, q_scale: float = 1.0,
                   kv_scale: float = 1.0, causal: bool = True, q_offset: int = 0, kv_offset: int = 0,
                   name: str = "") -> Fp8DenseCase:
    """q8 then kv8, each N(0, 1) / its scale quantised to e4m3 (so that the
    dequantised values are about N(0, 1) whatever the scales)."""
    rng = np.random.default_rng(seed)
    Nkv = N if Nkv is None else Nkv
    q8 = normal_e4m3(rng, (B, H, N, dk), std=1.0 / q_scale)
    kv8 = normal_e4m3(rng, (B, 1, Nkv, dk), std=1.0 / kv_scale)
    return Fp8DenseCase(q8, kv8, q_scale, kv_scale, dv, scale, causal, q_offset, kv_offset, name)


def dsv3_prefill_fp8(seed: int = 0) -> Fp8DenseCase:
    return fp8_dense_case(B=1, H=128, N=8192, seed=seed,
                          name="DeepSeek-V3 absorbed MLA prefill, FP8 e4m3 Q and KV, H=128 N=8192")
