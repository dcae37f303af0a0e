"""fp64 reference definitions.  TEST INFRASTRUCTURE ONLY (see package doc).

Arrays given as ``uint16`` are bfloat16 bit patterns and are widened exactly
to float64; float arrays are used as they are.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def _f64(x: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> float64 exactly; float arrays -> float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# ---------------------------------------------------------------------------
# softmax attention with log-sum-exp
# ---------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              causal: bool, q_pos: np.ndarray, k_pos: np.ndarray
              ) -> Tuple[np.ndarray, np.ndarray]:
    """One head: q [Nq, dk], k [Nk, dk], v [Nk, dv] -> (O [Nq, dv], lse [Nq]).

    Key j is visible to query i unless ``causal`` and k_pos[j] > q_pos[i]
    (positions are global sequence positions: the TRIU mask of Ascend
    ``maskType`` and the logical global length of TT-NN ``logical_n``).
    Scores are ``scale * q.k`` (``qkScale`` post-multiplies Q K^T).  LSE is
    the natural log of the sum of exp of the scaled visible scores; a row with
    no visible key gets O = 0 and LSE = -inf.
    """
    q = _f64(q); k = _f64(k); v = _f64(v)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    s = scale * (q @ k.T)                                   # [Nq, Nk]
    if causal:
        visible = k_pos[None, :] <= q_pos[:, None]
    else:
        visible = np.ones(s.shape, dtype=bool)
    s = np.where(visible, s, NEG_INF)
    any_vis = visible.any(axis=1)
    m = np.where(any_vis, s.max(axis=1, initial=NEG_INF), 0.0)   # pass 1: row max
    w = np.where(visible, np.exp(s - m[:, None]), 0.0)          # pass 2: weights
    l = w.sum(axis=1)
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    out[any_vis] = (w[any_vis] @ v) / l[any_vis, None]
    lse = np.full(q.shape[0], NEG_INF)
    lse[any_vis] = m[any_vis] + np.log(l[any_vis])
    return out, lse


def dense_mla(q: np.ndarray, kv: np.ndarray, head_dim_v: int, scale: float,
              causal: bool = True, q_offset: int = 0, kv_offset: int = 0,
              v: Optional[np.ndarray] = None,
              rows: Optional[Sequence[int]] = None,
              heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """q [B, Hq, Nq, dk], kv [B, Hkv, Nkv, dk] -> O [B, Hq, nr, dv], lse [B, Hq, nr].

    The key is the whole KV row (all dk columns); the value is its first
    ``head_dim_v`` columns unless an explicit ``v`` [B, Hkv, Nkv, dv] is given.
    Query head h reads KV head h // (Hq / Hkv).  Query row i sits at global
    position q_offset + i and key j at kv_offset + j.  ``rows``/``heads``
    restrict the computation to a subset of query rows / heads (the result
    has only those rows / heads, in the order given).
    """
    B, Hq, Nq, dk = q.shape
    Hkv, Nkv = kv.shape[1], kv.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if v is None and head_dim_v > kv.shape[3]:
        raise ValueError("head_dim_v exceeds the KV width")
    group = Hq // Hkv
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, dtype=np.int64)
    dv = head_dim_v
    out = np.zeros((B, len(heads), len(rows), dv))
    lse = np.zeros((B, len(heads), len(rows)))
    q_pos = q_offset + rows
    k_pos = kv_offset + np.arange(Nkv)
    for b in range(B):
        for hi, h in enumerate(heads):
            kvh = h // group
            k = kv[b, kvh]
            vv = (kv[b, kvh, :, :dv] if v is None else v[b, kvh])
            out[b, hi], lse[b, hi] = attention(q[b, h, rows], k, vv, scale, causal,
                                               q_pos, k_pos)
    return out, lse


# ---------------------------------------------------------------------------
# merge of partial results
# ---------------------------------------------------------------------------
def merge(out_a: np.ndarray, lse_a: np.ndarray, out_b: np.ndarray, lse_b: np.ndarray
          ) -> Tuple[np.ndarray, np.ndarray]:
    """Fold two partial results over disjoint key sets.

    lse = log(exp(lse_a) + exp(lse_b)); out = exp(lse_a - lse) out_a +
    exp(lse_b - lse) out_b.  ``out`` has one more trailing axis than ``lse``.
    A side whose LSE is -inf has no visible key and weight exactly 0, and its
    output is not multiplied at all (so a NaN there cannot leak); both -inf
    gives (0, -inf).
    """
    oa = _f64(out_a); ob = _f64(out_b)
    la = np.asarray(lse_a, dtype=np.float64); lb = np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(la, lb)
    out = np.zeros(np.broadcast(oa, ob).shape)
    for lx, ox in ((la, oa), (lb, ob)):
        live = ~np.isneginf(lx)
        w = np.exp(np.where(live, lx - np.where(live, lse, 0.0), NEG_INF))
        out[live] += w[live][..., None] * ox[live]
    return out, lse


# ---------------------------------------------------------------------------
# one-device ring over contiguous chunks
# ---------------------------------------------------------------------------
def ring_order(r: int, n_chunks: int):
    """KV chunks that query chunk r visits, in ring order: step s brings chunk
    (r - s) mod P, as each device of a ring receives its neighbour's KV in
    turn.  Chunks after r lie wholly in the causal future and contribute the
    fold identity (0, -inf), so they are skipped."""
    return [(r - s) % n_chunks for s in range(n_chunks) if (r - s) % n_chunks <= r]


def ring(q: np.ndarray, kv: np.ndarray, head_dim_v: int, scale: float, n_chunks: int,
         order=None,
         heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Causal attention of q [B,H,N,dk] over kv [B,1,N,dk] computed chunk by
    chunk: query chunk r attends each visited KV chunk k with global offsets
    (r*C, k*C) -- a FULL mask for k < r and the causal mask for k = r -- and
    each partial result is folded into the running (out, lse).  The first
    visit has no previous result.  ``order(r, P)`` may override the visiting
    order (any order of the same chunks gives the same result)."""
    B, H, N, dk = q.shape
    if N % n_chunks:
        raise ValueError("N must be a multiple of the chunk count")
    C = N // n_chunks
    order = order or ring_order
    heads = list(range(H)) if heads is None else list(heads)
    out = np.zeros((B, len(heads), N, head_dim_v))
    lse = np.full((B, len(heads), N), NEG_INF)
    qh = q[:, heads]
    for r in range(n_chunks):
        qs = slice(r * C, (r + 1) * C)
        acc_o = acc_l = None
        for k in order(r, n_chunks):
            ks = slice(k * C, (k + 1) * C)
            o, l = dense_mla(qh[:, :, qs], kv[:, :, ks], head_dim_v, scale, causal=True,
                             q_offset=r * C, kv_offset=k * C)
            if acc_o is None:
                acc_o, acc_l = o, l
            else:
                acc_o, acc_l = merge(acc_o, acc_l, o, l)
        out[:, :, qs], lse[:, :, qs] = acc_o, acc_l
    return out, lse


# ---------------------------------------------------------------------------
# split query/key ring step with per-sequence lengths
# ---------------------------------------------------------------------------
def split_mla(q1, q2, k1, k2, v, seq_lens, scale: float, causal: bool = True,
              prev_out=None, prev_lse=None,
              heads: Optional[Sequence[int]] = None,
              seqs: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Tokens of several sequences packed along axis 0 ([T, H, D] layouts).

    Ascend RingMLAOperation, member table (querySplit1/2, keySplit1/2, value,
    seqLen, maskType, prevOut/prevLse).  The score is scale * (q1.k1 + q2.k2):
    the query and key arrive split into the part without positional encoding
    and the rotary part.  V is separate.  ``seq_lens`` is either [batch]
    (sequence b owns the same token range [cu[b], cu[b] + len[b]) of the
    query and the key tensors) or [2, batch] (row 0 the query lengths, row 1
    the key lengths, each packed along its own tensor).  A query sees only
    keys of its own sequence; with ``causal`` (TRIU) the last query row and
    the last key row of a sequence share a position, so query i of a
    sequence with Lq queries and Lk keys sees key j iff j <= i + Lk - Lq
    (equal lengths: j <= i).  Query head h reads KV head h // (H / Hkv).
    With ``prev_out`` [Tq, H, dv] and ``prev_lse`` [H, Tq] the new result is
    folded into the previous one.  Returns out [Tq, H, dv] and lse [H, Tq]
    (restricted to ``heads``/``seqs`` when given: other entries are left as
    zeros / -inf).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    q_lens, k_lens = (seq_lens, seq_lens) if seq_lens.ndim == 1 else (seq_lens[0], seq_lens[1])
    T, H = q1.shape[0], q1.shape[1]
    Hkv = k1.shape[1]
    group = H // Hkv
    dv = v.shape[2]
    cq = np.concatenate([[0], np.cumsum(q_lens)])
    ck = np.concatenate([[0], np.cumsum(k_lens)])
    if cq[-1] != T or ck[-1] != k1.shape[0]:
        raise ValueError("sequence lengths do not add up to the token counts")
    heads = range(H) if heads is None else heads
    seqs = range(len(q_lens)) if seqs is None else seqs
    out = np.zeros((T, H, dv))
    lse = np.full((H, T), NEG_INF)
    for b in seqs:
        t0, t1 = int(cq[b]), int(cq[b + 1])
        u0, u1 = int(ck[b]), int(ck[b + 1])
        kpos = np.arange(u1 - u0)
        qpos = np.arange(t1 - t0) + (u1 - u0) - (t1 - t0)  # the last rows share a position
        for h in heads:
            kvh = h // group
            qq = np.concatenate([_f64(q1[t0:t1, h]), _f64(q2[t0:t1, h])], axis=1)
            kk = np.concatenate([_f64(k1[u0:u1, kvh]), _f64(k2[u0:u1, kvh])], axis=1)
            o, l = attention(qq, kk, _f64(v[u0:u1, kvh]), scale, causal, qpos, kpos)
            if prev_out is not None:
                o, l = merge(prev_out[t0:t1, h], prev_lse[h, t0:t1], o, l)
            out[t0:t1, h], lse[h, t0:t1] = o, l
    return out, lse


# ---------------------------------------------------------------------------
# sparse top-k latent attention
# ---------------------------------------------------------------------------
def sparse_mla(q_lift, q_pe, c_kv, k_pe, idx, scale: float,
               rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """q_lift [B,S,H,L], q_pe [B,S,H,R], c_kv [B,S_kv,L], k_pe [B,S_kv,R],
    idx int32 [B,S,K] -> out [B, nr, H*L] (column h*L + l), lse [B, nr, H].

    Query i of batch b attends exactly the K cache rows idx[b, i, :] (a
    multiset: a repeated index counts as often as it is listed; the order is
    irrelevant) with score scale * (q_lift . c_kv + q_pe . k_pe); the value is
    the latent row c_kv.  All heads of a query share its index list.  The
    pages leave indices outside [0, S_kv) undefined; here such an entry is
    not attended (like a -1 padding sentinel), and a query with no valid
    entry gets out = 0 and lse = -inf.
    """
    B, S, H, L = q_lift.shape
    S_kv = c_kv.shape[1]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, len(rows), H * L))
    lse = np.full((B, len(rows), H), NEG_INF)
    for b in range(B):
        for ri, i in enumerate(rows):
            sel = np.asarray(idx[b, i], dtype=np.int64)
            sel = sel[(sel >= 0) & (sel < S_kv)]
            if sel.size == 0:
                continue
            ck = _f64(c_kv[b, sel])                       # [K, L]
            kp = _f64(k_pe[b, sel])                       # [K, R]
            s = scale * (_f64(q_lift[b, i]) @ ck.T + _f64(q_pe[b, i]) @ kp.T)   # [H, K]
            m = s.max(axis=1)
            w = np.exp(s - m[:, None])
            l = w.sum(axis=1)
            out[b, ri] = ((w @ ck) / l[:, None]).reshape(-1)
            lse[b, ri] = m + np.log(l)
    return out, lse


def mx4_pack(out: np.ndarray, L: int) -> np.ndarray:
    """Sparse output [..., H*L] in natural column order -> the same values
    with each head's L columns in MX 4-pack order (NKI
    ``mla_sparse_attention_cte_kernel``, "Returns" and "Notes"): the value of
    natural latent column l = 4*group + sub lands at column sub*(L//4) + group
    of its head.  Written as the scatter the pages state, one column at a time.
    """
    if L % 4:
        raise ValueError("L must be a multiple of 4")
    lead = out.shape[:-1]
    H = out.shape[-1] // L
    nat = out.reshape(*lead, H, L)
    phys = np.empty_like(nat)
    for l in range(L):
        group, sub = divmod(l, 4)
        phys[..., sub * (L // 4) + group] = nat[..., l]
    return phys.reshape(out.shape)


# ---------------------------------------------------------------------------
# V-up projection of the latent output
# ---------------------------------------------------------------------------
def vup(o: np.ndarray, w_uv: np.ndarray, mx4: bool = False) -> np.ndarray:
    """o [B, H, T, L], w_uv [H, dvh, L] -> [B, H, T, dvh] with
    out[b, h, t, c] = sum_l o[b, h, t, l] * w_uv[h, c, l] (TensorRT-LLM
    ``mla.py``, ``forward_absorption_context``: the per-head product of the
    latent attention output [heads, tokens, kv_lora_rank] with ``v_b_proj``
    transposed).  ``mx4``: o's columns are in MX 4-pack order (see
    :func:`mx4_pack`); they are put back in natural order first.
    """
    o = _f64(o)
    L = o.shape[-1]
    if mx4:
        l = np.arange(L)
        o = o[..., (l % 4) * (L // 4) + l // 4]
    w = _f64(w_uv)
    out = np.empty(o.shape[:-1] + (w.shape[1],))
    for h in range(o.shape[1]):
        out[:, h] = o[:, h] @ w[h].T
    return out


# ---------------------------------------------------------------------------
# token generation: one new query per sequence over its valid cache rows
# ---------------------------------------------------------------------------
def decode_mla(q: np.ndarray, kv: np.ndarray, kv_lens: Optional[Sequence[int]],
               head_dim_v: int, scale: float,
               kv_slots: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """q [B, H, dk] (the newest token of each sequence), kv [n_slots, Nkv, dk],
    kv_lens [B] (None: Nkv for every sequence) -> out [B, H, dv], lse [B, H].

    kv_slots [B] (TT-NN ring_mla kv_cache_batch_idx: one batch slot of an
    indexed cache) names the cache slot sequence b reads; None reads slot b.
    A slot outside [0, n_slots) leaves the sequence without valid rows.

    Mojo mha_single_batch_pipelined (token generation, seq_len = 1, with
    num_keys valid cache entries per sequence): the query of sequence b is
    its newest token, so it sees its first kv_lens[b] cache rows, every one
    of them.  The key is the whole row and the value its first head_dim_v
    columns, as in dense_mla.  A sequence with no valid row gets out = 0 and
    lse = -inf.  Splitting the rows into ranges and folding the partial
    results (merge) gives the same result; that split over the keys is the
    page's split-K with its separate reduction.
    """
    B, H, dk = q.shape
    n_slots, Nkv = kv.shape[0], kv.shape[1]
    lens = [Nkv] * B if kv_lens is None else [int(x) for x in kv_lens]
    slots = list(range(B)) if kv_slots is None else [int(x) for x in kv_slots]
    out = np.zeros((B, H, head_dim_v))
    lse = np.full((B, H), NEG_INF)
    for b in range(B):
        n = max(0, min(Nkv, lens[b]))
        if n == 0 or not 0 <= slots[b] < n_slots:
            continue
        k = kv[slots[b], :n]
        o, l = attention(q[b], k, k[:, :head_dim_v], scale, causal=False,
                         q_pos=np.zeros(H, dtype=np.int64), k_pos=np.zeros(n, dtype=np.int64))
        out[b], lse[b] = o, l
    return out, lse
