"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against brute force on tiny inputs, a library
routine (torch's scaled_dot_product_attention in float64 on the CPU), closed
forms, the hand-worked fixture in ``tests/golden/hand_worked.json`` or an
invariant the method fixes (chunked-and-merged equals unchunked).  The last
group plants plausible mistakes in a copy of the oracle and checks that a pin
catches each of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_ref
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# brute force on tiny inputs
# ---------------------------------------------------------------------------
def brute_attention(q, k, v, scale, causal, q_pos, k_pos):
    """Literal softmax(scale Q K^T + M) V with Python loops, an explicit mask
    and no max subtraction (inputs are small, so exp cannot overflow)."""
    nq, nk, dv = len(q), len(k), len(v[0])
    out = [[0.0] * dv for _ in range(nq)]
    lse = [0.0] * nq
    for i in range(nq):
        weights = []
        for j in range(nk):
            if causal and k_pos[j] > q_pos[i]:
                weights.append(0.0)
                continue
            dot = 0.0
            for d in range(len(q[i])):
                dot += q[i][d] * k[j][d]
            weights.append(math.exp(scale * dot))
        z = sum(weights)
        if z == 0.0:
            lse[i] = -math.inf
            continue
        lse[i] = math.log(z)
        for c in range(dv):
            out[i][c] = sum(weights[j] * v[j][c] for j in range(nk)) / z
    return np.array(out), np.array(lse)


@pytest.mark.parametrize("q_off,kv_off,nq,nk", [(0, 0, 7, 7), (3, 0, 5, 9), (6, 4, 4, 6), (0, 2, 4, 5)])
def test_dense_matches_brute_force(q_off, kv_off, nq, nk):
    rng = np.random.default_rng(1)
    H, dk, dv = 3, 10, 6
    q = _rand(rng, 1, H, nq, dk)
    kv = _rand(rng, 1, 1, nk, dk)
    scale = 0.37
    out, lse = oracle.dense_mla(q, kv, dv, scale, causal=True, q_offset=q_off, kv_offset=kv_off)
    for h in range(H):
        bo, bl = brute_attention(q[0, h].tolist(), kv[0, 0].tolist(), kv[0, 0, :, :dv].tolist(),
                                 scale, True, list(range(q_off, q_off + nq)),
                                 list(range(kv_off, kv_off + nk)))
        np.testing.assert_allclose(out[0, h], bo, rtol=0, atol=1e-12)
        fin = np.isfinite(bl)
        assert np.array_equal(fin, np.isfinite(lse[0, h]))
        np.testing.assert_allclose(lse[0, h][fin], bl[fin], rtol=0, atol=1e-12)


def test_dense_noncausal_matches_brute_force():
    rng = np.random.default_rng(2)
    q = _rand(rng, 1, 2, 5, 8)
    kv = _rand(rng, 1, 1, 6, 8)
    out, lse = oracle.dense_mla(q, kv, 4, 0.5, causal=False)
    for h in range(2):
        bo, bl = brute_attention(q[0, h].tolist(), kv[0, 0].tolist(), kv[0, 0, :, :4].tolist(),
                                 0.5, False, [0] * 5, [0] * 6)
        np.testing.assert_allclose(out[0, h], bo, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], bl, atol=1e-12)


# ---------------------------------------------------------------------------
# library routine: torch scaled_dot_product_attention in float64 (CPU)
# ---------------------------------------------------------------------------
def test_dense_matches_sdpa_float64():
    rng = np.random.default_rng(3)
    B, H, N, dk, dv = 2, 4, 64, 40, 32
    q = _rand(rng, B, H, N, dk)
    kv = _rand(rng, B, 1, N, dk)
    scale = 1 / math.sqrt(192)
    out, _ = oracle.dense_mla(q, kv, dv, scale, causal=True)
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(kv).expand(B, H, N, dk)
    tv = torch.from_numpy(kv[..., :dv].copy()).expand(B, H, N, dv)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_grouped_heads_match_sdpa_float64():
    rng = np.random.default_rng(4)
    B, H, Hkv, N, dk, dv = 1, 6, 2, 24, 16, 16
    q = _rand(rng, B, H, N, dk)
    kv = _rand(rng, B, Hkv, N, dk)
    v = _rand(rng, B, Hkv, N, dv)
    out, _ = oracle.dense_mla(q, kv, dv, 0.3, causal=True, v=v)
    tk = torch.from_numpy(kv).repeat_interleave(H // Hkv, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(H // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), tk, tv,
                                                           is_causal=True, scale=0.3)
    np.testing.assert_allclose(out, ref.numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_first_row_closed_form():
    """Query 0 at offset 0 sees only key 0: O = V_0 and LSE = scale q_0.k_0."""
    c = W.dense_case(B=1, H=3, N=16, dk=576, dv=512, seed=5)
    out, lse = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    q = W.bf16_bits_to_f64(c.q); kv = W.bf16_bits_to_f64(c.kv)
    for h in range(3):
        np.testing.assert_array_equal(out[0, h, 0], kv[0, 0, 0, :512])
        assert abs(lse[0, h, 0] - c.scale * float(np.dot(q[0, h, 0], kv[0, 0, 0]))) < 1e-12


@pytest.mark.parametrize("q_off,kv_off,nq,nk", [(0, 0, 12, 12), (5, 2, 6, 10), (10, 0, 3, 16), (3, 7, 8, 6)])
def test_zero_scale_gives_prefix_mean(q_off, kv_off, nq, nk):
    """scale = 0 makes every visible weight equal: O is the mean of the visible
    V rows and LSE = ln(#visible); this pins the mask boundary exactly."""
    rng = np.random.default_rng(6)
    q = _rand(rng, 1, 2, nq, 12)
    kv = _rand(rng, 1, 1, nk, 12)
    out, lse = oracle.dense_mla(q, kv, 8, 0.0, q_offset=q_off, kv_offset=kv_off)
    for i in range(nq):
        n_vis = sum(1 for j in range(nk) if kv_off + j <= q_off + i)
        if n_vis == 0:
            assert np.all(out[0, :, i] == 0) and np.all(np.isneginf(lse[0, :, i]))
            continue
        mean = kv[0, 0, :n_vis, :8].mean(axis=0)
        for h in range(2):
            np.testing.assert_allclose(out[0, h, i], mean, atol=1e-13)
            assert abs(lse[0, h, i] - math.log(n_vis)) < 1e-13


def test_identical_keys_closed_form():
    """All KV rows equal: O = that V row; LSE = s + ln(#visible)."""
    rng = np.random.default_rng(7)
    row = _rand(rng, 20)
    kv = np.tile(row, (1, 1, 9, 1))
    q = _rand(rng, 1, 2, 9, 20)
    out, lse = oracle.dense_mla(q, kv, 16, 0.25)
    for h in range(2):
        for i in range(9):
            np.testing.assert_allclose(out[0, h, i], row[:16], atol=1e-13)
            s = 0.25 * float(q[0, h, i] @ row)
            assert abs(lse[0, h, i] - (s + math.log(i + 1))) < 1e-12


def test_fully_masked_rows():
    rng = np.random.default_rng(8)
    q = _rand(rng, 1, 1, 4, 8)
    kv = _rand(rng, 1, 1, 4, 8)
    out, lse = oracle.dense_mla(q, kv, 4, 1.0, q_offset=0, kv_offset=4)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_explicit_prefix_value_is_identical():
    """V = KV[..., :dv] read from the KV rows equals passing that slice as V."""
    c = W.dense_case(B=1, H=2, N=40, seed=9)
    a = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    b = oracle.dense_mla(c.q, c.kv, 512, c.scale, v=c.kv[..., :512].copy())
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# hand-worked golden values
# ---------------------------------------------------------------------------
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_dense():
    g = _golden()["dense"]
    vcols = np.array(g["kv_value_cols"], float)
    scol = np.log(np.array(g["kv_score_col_exp"], float))
    kv = np.concatenate([vcols, scol[:, None]], axis=1)[None, None]
    q = np.array(g["q"], float)[None, None]
    out, lse = oracle.dense_mla(q, kv, g["head_dim_v"], g["scale"])
    np.testing.assert_allclose(out[0, 0], np.array(g["out"]), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(g["lse_exp"]), atol=1e-14)


def test_golden_merge():
    g = _golden()["merge"]
    o, l = oracle.merge(np.array([g["out_a"]], float), np.array([math.log(g["lse_a_exp"])]),
                        np.array([g["out_b"]], float), np.array([math.log(g["lse_b_exp"])]))
    np.testing.assert_allclose(o[0], g["out"], atol=1e-14)
    assert abs(l[0] - math.log(g["lse_exp"])) < 1e-14


def test_golden_sparse():
    g = _golden()["sparse"]
    dense = _golden()["dense"]
    c_kv = np.array(dense["kv_value_cols"], float)[None]
    k_pe = np.log(np.array(dense["kv_score_col_exp"], float))[None, :, None]
    q_lift = np.zeros((1, 1, 1, 2)); q_pe = np.ones((1, 1, 1, 1))
    idx = np.array(g["idx"], np.int32)[None, None]
    out, lse = oracle.sparse_mla(q_lift, q_pe, c_kv, k_pe, idx, 1.0)
    np.testing.assert_allclose(out[0, 0], g["out"], atol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(g["lse_exp"])) < 1e-14


def test_golden_split():
    g = _golden()["split"]
    ln2, ln3 = math.log(2), math.log(3)
    q1 = np.array([[[1, 0]], [[1, 0]]], float); q2 = np.array([[[0]], [[1]]], float)
    k1 = np.array([[[ln2, 5]], [[0, 7]]]); k2 = np.array([[[0]], [[ln3]]])
    v = np.array([[[4]], [[10]]], float)
    out, lse = oracle.split_mla(q1, q2, k1, k2, v, [2], 1.0)
    np.testing.assert_allclose(out[:, 0, 0], g["out"], atol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(g["lse_exp"]), atol=1e-14)


# ---------------------------------------------------------------------------
# merge and ring invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_chunks", [1, 2, 4, 8])
def test_ring_equals_unchunked(n_chunks):
    c = W.dense_case(B=1, H=2, N=64, dk=24, dv=16, seed=10, scale=0.3)
    o_full, l_full = oracle.dense_mla(c.q, c.kv, 16, 0.3)
    o_ring, l_ring = oracle.ring(c.q, c.kv, 16, 0.3, n_chunks)
    np.testing.assert_allclose(o_ring, o_full, atol=1e-12)
    np.testing.assert_allclose(l_ring, l_full, atol=1e-12)


def test_ring_any_order_equals_unchunked():
    c = W.dense_case(B=1, H=2, N=48, dk=24, dv=16, seed=11, scale=0.3)
    o_full, l_full = oracle.dense_mla(c.q, c.kv, 16, 0.3)
    rng = np.random.default_rng(0)

    def shuffled(r, P):
        ks = list(range(r + 1))
        rng.shuffle(ks)
        return ks

    o_ring, l_ring = oracle.ring(c.q, c.kv, 16, 0.3, 6, order=shuffled)
    np.testing.assert_allclose(o_ring, o_full, atol=1e-12)
    np.testing.assert_allclose(l_ring, l_full, atol=1e-12)


def test_ring_order_visits_each_past_chunk_once():
    for P in range(1, 9):
        for r in range(P):
            ks = oracle.ring_order(r, P)
            assert ks[0] == r and sorted(ks) == list(range(r + 1))


def test_merge_commutative_associative_identity():
    rng = np.random.default_rng(12)
    o = [_rand(rng, 5, 7) for _ in range(3)]
    lse = [_rand(rng, 5) * 3 for _ in range(3)]
    ab = oracle.merge(o[0], lse[0], o[1], lse[1])
    ba = oracle.merge(o[1], lse[1], o[0], lse[0])
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-14)
    np.testing.assert_allclose(ab[1], ba[1], atol=1e-14)
    left = oracle.merge(ab[0], ab[1], o[2], lse[2])
    bc = oracle.merge(o[1], lse[1], o[2], lse[2])
    right = oracle.merge(o[0], lse[0], bc[0], bc[1])
    np.testing.assert_allclose(left[0], right[0], atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], atol=1e-13)
    ident = oracle.merge(o[0], lse[0], np.full_like(o[1], np.nan), np.full(5, -np.inf))
    np.testing.assert_array_equal(ident[0], o[0])
    np.testing.assert_array_equal(ident[1], lse[0])


def test_merge_both_empty_is_nan_free():
    o, l = oracle.merge(np.full((3, 4), np.nan), np.full(3, -np.inf),
                        np.full((3, 4), np.nan), np.full(3, -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_merge_of_split_keys_equals_whole():
    """Attention over keys A u B equals the merge of attention over A and
    over B, for an arbitrary (non-contiguous) split of the keys."""
    rng = np.random.default_rng(13)
    q = _rand(rng, 6, 10); k = _rand(rng, 11, 10); v = _rand(rng, 11, 5)
    mask = rng.random(11) < 0.5
    pos0 = np.zeros(6, int)
    whole = oracle.attention(q, k, v, 0.4, False, pos0, np.zeros(11, int))
    a = oracle.attention(q, k[mask], v[mask], 0.4, False, pos0, np.zeros(mask.sum(), int))
    b = oracle.attention(q, k[~mask], v[~mask], 0.4, False, pos0, np.zeros((~mask).sum(), int))
    m = oracle.merge(a[0], a[1], b[0], b[1])
    np.testing.assert_allclose(m[0], whole[0], atol=1e-13)
    np.testing.assert_allclose(m[1], whole[1], atol=1e-13)


# ---------------------------------------------------------------------------
# sparse top-k
# ---------------------------------------------------------------------------
def _small_sparse(seed=14, S=6, S_kv=40, pos0=30, H=3, L=16, R=8, K=12):
    return W.sparse_case(S=S, S_kv=S_kv, pos0=pos0, H=H, L=L, R=R, K=K, seed=seed, scale=0.2)


def test_sparse_all_causal_rows_equals_dense_row():
    c = _small_sparse()
    pos = int(c.positions[2])
    idx = np.arange(pos + 1, dtype=np.int32)[None, None]
    out, lse = oracle.sparse_mla(c.q_lift[:, 2:3], c.q_pe[:, 2:3], c.c_kv, c.k_pe, idx, c.scale)
    # dense form: q = [q_lift | q_pe] per head, one KV head = [c_kv | k_pe], V = c_kv
    q = np.concatenate([W.bf16_bits_to_f64(c.q_lift[0, 2]), W.bf16_bits_to_f64(c.q_pe[0, 2])], axis=1)
    kv = np.concatenate([W.bf16_bits_to_f64(c.c_kv[0]), W.bf16_bits_to_f64(c.k_pe[0])], axis=1)
    o_d, l_d = oracle.dense_mla(q[None, :, None, :], kv[None, None], 16, c.scale,
                                q_offset=pos, kv_offset=0)
    np.testing.assert_allclose(out[0, 0].reshape(3, 16), o_d[0, :, 0], atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], l_d[0, :, 0], atol=1e-12)


def test_sparse_permutation_invariant():
    c = _small_sparse()
    rng = np.random.default_rng(0)
    perm = c.idx.copy()
    for i in range(perm.shape[1]):
        rng.shuffle(perm[0, i])
    a = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, c.idx, c.scale)
    b = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, perm, c.scale)
    np.testing.assert_allclose(a[0], b[0], atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], atol=1e-12)


def test_sparse_repeated_row_closed_form():
    """K copies of row r: p = 1/K, out = c_kv[r] exactly, LSE = s_r + ln K."""
    c = _small_sparse()
    K, r = 12, 17
    idx = np.full((1, c.idx.shape[1], K), r, np.int32)
    out, lse = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, idx, c.scale)
    crow = W.bf16_bits_to_f64(c.c_kv[0, r]); prow = W.bf16_bits_to_f64(c.k_pe[0, r])
    for i in range(idx.shape[1]):
        for h in range(3):
            np.testing.assert_allclose(out[0, i, h * 16:(h + 1) * 16], crow, atol=1e-14)
            s = c.scale * (W.bf16_bits_to_f64(c.q_lift[0, i, h]) @ crow
                           + W.bf16_bits_to_f64(c.q_pe[0, i, h]) @ prow)
            assert abs(lse[0, i, h] - (s + math.log(K))) < 1e-12


def test_sparse_indices_distinct_and_causal():
    c = _small_sparse()
    for i in range(c.idx.shape[1]):
        row = c.idx[0, i]
        assert len(set(row.tolist())) == len(row)
        assert row.min() >= 0 and row.max() <= c.positions[i]


def test_sparse_out_of_range_index_is_skipped():
    """An index outside [0, S_kv) is not attended: the result equals the one
    without that entry; a list with no valid entry gives (0, -inf)."""
    c = _small_sparse()
    bad = c.idx.copy()
    bad[0, 0, 0] = c.c_kv.shape[1]
    bad[0, 1, 3] = -1
    a = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, bad, c.scale, rows=[0, 1])
    r0 = oracle.sparse_mla(c.q_lift[:, 0:1], c.q_pe[:, 0:1], c.c_kv, c.k_pe, c.idx[:, 0:1, 1:], c.scale)
    keep = [j for j in range(c.idx.shape[2]) if j != 3]
    r1 = oracle.sparse_mla(c.q_lift[:, 1:2], c.q_pe[:, 1:2], c.c_kv, c.k_pe, c.idx[:, 1:2, keep], c.scale)
    np.testing.assert_allclose(a[0][:, 0], r0[0][:, 0], atol=1e-13)
    np.testing.assert_allclose(a[0][:, 1], r1[0][:, 0], atol=1e-13)
    none = np.full_like(c.idx[:, :1], -1)
    o, l = oracle.sparse_mla(c.q_lift[:, :1], c.q_pe[:, :1], c.c_kv, c.k_pe, none, c.scale)
    assert np.all(o == 0) and np.all(np.isneginf(l))


# ---------------------------------------------------------------------------
# split q/k varlen step
# ---------------------------------------------------------------------------
def test_split_matches_sdpa_per_sequence():
    c = W.split_case(seq_lens=[5, 9, 1, 7], H=4, Hkv=2, d_nope=16, d_rope=8, dv=12, seed=15)
    out, lse = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale)
    cu = np.concatenate([[0], np.cumsum(c.seq_lens)])
    f = W.bf16_bits_to_f64
    for b in range(4):
        t0, t1 = cu[b], cu[b + 1]
        q = torch.from_numpy(np.concatenate([f(c.q1[t0:t1]), f(c.q2[t0:t1])], -1)).permute(1, 0, 2)
        k = torch.from_numpy(np.concatenate([f(c.k1[t0:t1]), f(c.k2[t0:t1])], -1)).permute(1, 0, 2)
        v = torch.from_numpy(f(c.v[t0:t1])).permute(1, 0, 2)
        k = k.repeat_interleave(2, dim=0); v = v.repeat_interleave(2, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=c.scale)
        np.testing.assert_allclose(out[t0:t1], ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_split_prev_fold_is_merge():
    c = W.split_case(seq_lens=[6, 3], H=2, Hkv=2, d_nope=8, d_rope=4, dv=8, seed=16)
    fresh = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale)
    folded = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale,
                              prev_out=c.prev_out, prev_lse=c.prev_lse)
    m = oracle.merge(c.prev_out, c.prev_lse.T, fresh[0], fresh[1].T)
    np.testing.assert_allclose(folded[0], m[0], atol=1e-13)
    np.testing.assert_allclose(folded[1], m[1].T, atol=1e-13)
    # an empty previous result (-inf) leaves the fresh result unchanged
    empty = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale,
                             prev_out=c.prev_out, prev_lse=np.full_like(c.prev_lse, -np.inf))
    np.testing.assert_allclose(empty[0], fresh[0], atol=1e-15)
    np.testing.assert_allclose(empty[1], fresh[1], atol=1e-15)


def _split_cat(c, toks, heads_of, which):
    """Rows ``toks`` of the split tensors joined into whole vectors (q: q1|q2
    of the given heads; k: k1|k2; v)."""
    f = W.bf16_bits_to_f64
    if which == "q":
        return np.concatenate([f(c.q1[toks][:, heads_of]), f(c.q2[toks][:, heads_of])], -1)
    if which == "k":
        return np.concatenate([f(c.k1[toks][:, heads_of]), f(c.k2[toks][:, heads_of])], -1)
    return f(c.v[toks][:, heads_of])


def test_split_two_row_lengths_brute_force():
    """[2, batch] lengths (Ascend seqLen, second form): sequence b's queries
    come from its own range of the query tensor, its keys from its own range
    of the key tensors; under TRIU the last query and the last key of a
    sequence share a position.  Pure-Python loops over every (query, key)
    pair, including sequences with fewer keys than queries (their first
    queries see no key) and with no keys or no queries at all."""
    ql, kl = [3, 5, 0, 4, 2], [6, 2, 3, 4, 0]
    c = W.split_case(seq_lens=ql, kv_lens=kl, H=2, Hkv=1, d_nope=8, d_rope=4, dv=6, seed=31)
    for causal in (True, False):
        out, lse = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale, causal=causal)
        tq = tk = 0
        for Lq, Lk in zip(ql, kl):
            for h in range(2):
                for i in range(Lq):
                    q = _split_cat(c, [tq + i], [h], "q")[0, 0]
                    vis = [j for j in range(Lk) if not causal or j <= i + Lk - Lq]
                    if not vis:
                        assert np.all(out[tq + i, h] == 0) and np.isneginf(lse[h, tq + i])
                        continue
                    s = [c.scale * float(q @ _split_cat(c, [tk + j], [0], "k")[0, 0]) for j in vis]
                    m = max(s)
                    w = [math.exp(x - m) for x in s]
                    o = sum(wj * _split_cat(c, [tk + j], [0], "v")[0, 0] for wj, j in zip(w, vis)) / sum(w)
                    np.testing.assert_allclose(out[tq + i, h], o, atol=1e-12)
                    assert abs(lse[h, tq + i] - (m + math.log(sum(w)))) < 1e-12
            tq += Lq
            tk += Lk


def test_split_two_row_equal_lengths_is_one_row():
    c = W.split_case(seq_lens=[4, 7, 2], H=2, Hkv=2, d_nope=8, d_rope=4, dv=8, seed=32)
    one = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale)
    two = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, np.stack([c.seq_lens, c.seq_lens]), c.scale)
    assert np.array_equal(one[0], two[0]) and np.array_equal(one[1], two[1])


def _chunk_of(c, lens, parts):
    """Per sequence, the token ranges of the chunks ``parts`` ([(start, stop)]
    within the sequence) gathered from the packed tensors."""
    cu = np.concatenate([[0], np.cumsum(lens)])
    return [int(cu[b]) + t for b, (a, z) in enumerate(parts) for t in range(a, z)]


def test_split_ring_step_over_a_past_chunk():
    """The Ascend ring on split tensors: each sequence's current chunk of
    queries meets an earlier chunk of keys with no mask (a non-first card's
    step, [2, batch] lengths), then its own chunk under TRIU with the first
    result as prevOut/prevLse.  Folded, the two steps give the rows of the
    plain causal call over the whole sequences, restricted to the current
    chunk."""
    lens = [9, 6, 11]
    whole = W.split_case(seq_lens=lens, H=2, Hkv=1, d_nope=8, d_rope=4, dv=6, seed=33, with_prev=False)
    ref_o, ref_l = oracle.split_mla(whole.q1, whole.q2, whole.k1, whole.k2, whole.v, whole.seq_lens,
                                    whole.scale)
    past = [(0, 4), (0, 2), (0, 7)]   # each sequence's earlier chunk
    cur = [(4, 9), (2, 6), (7, 11)]   # and its current one
    qt, kt = _chunk_of(whole, lens, cur), _chunk_of(whole, lens, past)
    ql = [z - a for a, z in cur]
    kl = [z - a for a, z in past]
    sub = lambda x, t: x[t]
    o1, l1 = oracle.split_mla(sub(whole.q1, qt), sub(whole.q2, qt), sub(whole.k1, kt), sub(whole.k2, kt),
                              sub(whole.v, kt), np.stack([ql, kl]), whole.scale, causal=False)
    o2, l2 = oracle.split_mla(sub(whole.q1, qt), sub(whole.q2, qt), sub(whole.k1, qt), sub(whole.k2, qt),
                              sub(whole.v, qt), ql, whole.scale, causal=True, prev_out=o1, prev_lse=l1)
    np.testing.assert_allclose(o2, ref_o[qt], atol=1e-12)
    np.testing.assert_allclose(l2, ref_l[:, qt], atol=1e-12)


def test_split_two_row_causal_is_chunked_prefill():
    """Queries of each sequence's last chunk against the keys of the whole
    sequence so far, under TRIU with [2, batch] lengths: the rows of the plain
    causal call over the whole sequences (TensorRT-LLM chunked prefill: a new
    chunk attends its cached prefix and itself causally).  Pins the alignment
    of the last rows."""
    lens = [8, 5, 12, 3]
    whole = W.split_case(seq_lens=lens, H=4, Hkv=2, d_nope=8, d_rope=4, dv=6, seed=34, with_prev=False)
    ref_o, ref_l = oracle.split_mla(whole.q1, whole.q2, whole.k1, whole.k2, whole.v, whole.seq_lens,
                                    whole.scale)
    cur = [(5, 8), (0, 5), (9, 12), (2, 3)]
    qt = _chunk_of(whole, lens, cur)
    ql = [z - a for a, z in cur]
    o, l = oracle.split_mla(whole.q1[qt], whole.q2[qt], whole.k1, whole.k2, whole.v, np.stack([ql, lens]),
                            whole.scale, causal=True)
    np.testing.assert_allclose(o, ref_o[qt], atol=1e-12)
    np.testing.assert_allclose(l, ref_l[:, qt], atol=1e-12)


def test_split_default_draw_lengths():
    """The seeded length draw of the 8-sequence workload (uniform in
    [1024, 8192])."""
    rng = np.random.default_rng(0)
    lens = rng.integers(1024, 8192, 8, endpoint=True)
    assert lens.min() >= 1024 and lens.max() <= 8192
    assert int(lens.sum()) == 27610


def test_mx4_pack_hand_worked():
    """The MX 4-pack column order on the hand-worked L = 8, H = 2 example."""
    g = json.load(open(GOLDEN))["mx4"]
    got = oracle.mx4_pack(np.array(g["natural"], dtype=np.float64)[None], g["L"])
    np.testing.assert_array_equal(got[0], np.array(g["physical"], dtype=np.float64))


def test_mx4_pack_is_a_per_head_permutation():
    """At L = 512: every head's columns are a permutation of its own columns,
    natural column 4g + s sits at s*128 + g, and the four subs of a group land
    in the four quarters of the head."""
    H, L = 3, 512
    nat = np.arange(H * L, dtype=np.float64).reshape(1, 1, H * L)
    phys = oracle.mx4_pack(nat, L).reshape(H, L)
    for h in range(H):
        assert sorted(phys[h]) == list(range(h * L, (h + 1) * L))
    l = np.arange(L)
    np.testing.assert_array_equal(phys[:, (l % 4) * (L // 4) + l // 4], nat.reshape(H, L))
    np.testing.assert_array_equal(phys[0, :4], [0, 4, 8, 12])
    np.testing.assert_array_equal(phys[0, 128:132], [1, 5, 9, 13])


# ---------------------------------------------------------------------------
# weight absorption: latent form == per-head form
# ---------------------------------------------------------------------------
def test_absorbed_equals_non_absorbed():
    """With W_UK, W_UV [H, d_nope, L]: attention with q_lift = q_nope W_UK_h
    over the shared latent rows [c_kv | k_pe] (value c_kv), followed by the
    V-up projection by W_UV_h, equals per-head attention with
    k_nope = c_kv W_UK_h^T and v = c_kv W_UV_h^T (TensorRT-LLM mla.py,
    forward_absorption_context / forward_absorption_generation)."""
    rng = np.random.default_rng(17)
    H, N, dn, dr, L, dvh = 3, 10, 8, 4, 12, 6
    q_nope = _rand(rng, N, H, dn); q_pe = _rand(rng, N, H, dr)
    c_kv = _rand(rng, N, L); k_pe = _rand(rng, N, dr)
    w_uk = _rand(rng, H, dn, L); w_uv = _rand(rng, H, dvh, L)
    scale = 1 / math.sqrt(dn + dr)
    q_lift = np.einsum("nhd,hdl->hnl", q_nope, w_uk)
    q_abs = np.concatenate([q_lift, q_pe.transpose(1, 0, 2)], -1)[None]
    kv = np.concatenate([c_kv, k_pe], -1)[None, None]
    o_lat, l_lat = oracle.dense_mla(q_abs, kv, L, scale)
    o_abs = oracle.vup(o_lat, w_uv)[0].transpose(1, 0, 2)
    k_nope = np.einsum("nl,hdl->nhd", c_kv, w_uk)
    v = np.einsum("nl,hvl->nhv", c_kv, w_uv)
    k_pe_h = np.repeat(k_pe[:, None, :], H, axis=1)
    o_per, l_per = oracle.split_mla(q_nope, q_pe, k_nope, k_pe_h, v, [N], scale)
    np.testing.assert_allclose(o_abs, o_per, atol=1e-10)
    np.testing.assert_allclose(l_lat[0], l_per, atol=1e-10)


def test_vup_brute_force():
    """V-up with Python loops over every (b, h, t, c) on a tiny case."""
    rng = np.random.default_rng(18)
    B, H, T, L, dvh = 2, 3, 4, 8, 5
    o = _rand(rng, B, H, T, L); w = _rand(rng, H, dvh, L)
    got = oracle.vup(o, w)
    for b, h, t, c in itertools.product(range(B), range(H), range(T), range(dvh)):
        want = sum(float(o[b, h, t, l]) * float(w[h, c, l]) for l in range(L))
        assert abs(got[b, h, t, c] - want) < 1e-12


def test_vup_commutes_with_merge():
    """Folding two partial results and then projecting equals projecting each
    and folding with the same LSE weights (TensorRT-LLM mla.py,
    _helix_project_v_partials: the combine is a per-head weighted sum, so it
    commutes with the per-head V projection)."""
    rng = np.random.default_rng(19)
    B, H, T, L, dvh = 1, 3, 5, 16, 4
    oa, ob = _rand(rng, B, H, T, L), _rand(rng, B, H, T, L)
    la, lb = _rand(rng, B, H, T), _rand(rng, B, H, T)
    la[0, 1, 2] = -np.inf
    w = _rand(rng, H, dvh, L)
    o_m, l_m = oracle.merge(oa, la, ob, lb)
    p_m, l_p = oracle.merge(oracle.vup(oa, w), la, oracle.vup(ob, w), lb)
    np.testing.assert_allclose(oracle.vup(o_m, w), p_m, atol=1e-12)
    np.testing.assert_array_equal(l_m, l_p)


def test_vup_mx4_input_equals_natural():
    """V-up of an MX 4-pack ordered input (mx4=True) equals V-up of the
    natural-order input, and treating the packed input as natural does not."""
    rng = np.random.default_rng(20)
    o = _rand(rng, 1, 2, 3, 16); w = _rand(rng, 2, 4, 16)
    packed = oracle.mx4_pack(o, 16)
    np.testing.assert_allclose(oracle.vup(packed, w, mx4=True), oracle.vup(o, w), atol=1e-12)
    assert np.abs(oracle.vup(packed, w) - oracle.vup(o, w)).max() > 1e-3


# ---------------------------------------------------------------------------
# token generation (decode)
# ---------------------------------------------------------------------------
def test_decode_matches_brute_force():
    rng = np.random.default_rng(60)
    B, H, N, dk, dv = 3, 2, 6, 5, 3
    q = _rand(rng, B, H, dk)
    kv = _rand(rng, B, N, dk)
    lens = [6, 3, 0]
    out, lse = oracle.decode_mla(q, kv, lens, dv, 0.7)
    for b in range(B):
        n = lens[b]
        o_bf, l_bf = brute_attention(q[b].tolist(), kv[b, :n].tolist(), kv[b, :n, :dv].tolist() or [[0.0] * dv],
                                     0.7, False, [0] * H, [0] * n)
        if n == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
        else:
            np.testing.assert_allclose(out[b], o_bf, atol=1e-12)
            np.testing.assert_allclose(lse[b], l_bf, atol=1e-12)


@pytest.mark.parametrize("L", [1, 17, 40])
def test_decode_is_last_row_of_causal_prefill(L):
    """The newest token's decode over the first L rows equals row L-1 of the
    causal prefill over those rows."""
    c = W.dense_case(B=1, H=3, N=40, seed=61)
    o_pre, l_pre = oracle.dense_mla(c.q[:, :, :L], c.kv[:, :, :L], 512, c.scale)
    q_new = np.ascontiguousarray(c.q[:, :, L - 1])             # [1, H, dk]
    kv_rows = np.ascontiguousarray(c.kv[:, 0])                  # [1, N, dk]
    o_dec, l_dec = oracle.decode_mla(q_new, kv_rows, [L], 512, c.scale)
    np.testing.assert_allclose(o_dec[0], o_pre[0, :, L - 1], atol=1e-12)
    np.testing.assert_allclose(l_dec[0], l_pre[0, :, L - 1], atol=1e-12)


def test_decode_zero_scale_prefix_mean():
    """scale 0: every visible weight is 1, so out is the mean of the first
    len value rows and lse = ln(len)."""
    rng = np.random.default_rng(62)
    q = _rand(rng, 2, 4, 9)
    kv = _rand(rng, 2, 30, 9)
    out, lse = oracle.decode_mla(q, kv, [30, 11], 6, 0.0)
    for b, n in enumerate([30, 11]):
        np.testing.assert_allclose(out[b], np.broadcast_to(kv[b, :n, :6].mean(axis=0), (4, 6)), atol=1e-12)
        np.testing.assert_allclose(lse[b], np.full(4, math.log(n)), atol=1e-12)


@pytest.mark.parametrize("cut", [0, 1, 700, 1999, 2000])
def test_decode_split_keys_merge_to_whole(cut):
    """Split-K: the rows [0, cut) and [cut, len) folded through their LSE
    give the whole result (an empty side is the fold identity)."""
    rng = np.random.default_rng(63)
    q = W.normal_bf16(rng, (2, 4, 576))
    kv = W.normal_bf16(rng, (2, 2000, 576))
    scale = W.SCALE_192
    whole = oracle.decode_mla(q, kv, [2000, 2000], 512, scale)
    a = oracle.decode_mla(q, kv, [cut, cut], 512, scale)
    b = oracle.decode_mla(q, np.ascontiguousarray(kv[:, cut:]), [2000 - cut] * 2, 512, scale)
    o, l = oracle.merge(a[0], a[1], b[0], b[1])
    np.testing.assert_allclose(o, whole[0], atol=1e-12)
    np.testing.assert_allclose(l, whole[1], atol=1e-12)


def test_decode_slots_select_cache_rows():
    """kv_slots: sequence b reads cache slot kv_slots[b]; the same as decoding
    against the cache rearranged so that slot b holds that slot; a slot out of
    range gives (0, -inf)."""
    rng = np.random.default_rng(64)
    q = _rand(rng, 4, 3, 7)
    kv = _rand(rng, 5, 20, 7)
    slots, lens = [3, 0, 3, 9], [20, 6, 11, 20]
    out, lse = oracle.decode_mla(q, kv, lens, 4, 0.6, kv_slots=slots)
    ref_o, ref_l = oracle.decode_mla(q[:3], kv[[3, 0, 3]], lens[:3], 4, 0.6)
    np.testing.assert_array_equal(out[:3], ref_o)
    np.testing.assert_array_equal(lse[:3], ref_l)
    assert np.all(out[3] == 0) and np.all(np.isneginf(lse[3]))


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# ---------------------------------------------------------------------------
def _mutant_attention(kind):
    orig = mla_ref.attention

    def mutant(q, k, v, scale, causal, q_pos, k_pos):
        if kind == "strict_mask":            # k_pos < q_pos instead of <=
            q_pos = np.asarray(q_pos) - 1
        elif kind == "drop_rope_cols":       # score over the first 512 columns only
            d = min(q.shape[1], 8)
            q = np.asarray(q)[:, :d]; k = np.asarray(k)[:, :d]
        elif kind == "lse_no_max":           # LSE forgets the subtracted max
            o, l = orig(q, k, v, scale, causal, q_pos, k_pos)
            s = scale * (mla_ref._f64(q) @ mla_ref._f64(k).T)
            return o, l - np.max(s, axis=1)
        elif kind == "value_suffix":         # V = last dv columns
            pass
        return orig(q, k, v, scale, causal, q_pos, k_pos)
    return mutant


@pytest.mark.parametrize("kind,pin", [
    ("strict_mask", test_zero_scale_gives_prefix_mean),
    ("drop_rope_cols", test_dense_matches_sdpa_float64),
    ("lse_no_max", test_first_row_closed_form),
])
def test_planted_mistake_is_caught(monkeypatch, kind, pin):
    monkeypatch.setattr(mla_ref, "attention", _mutant_attention(kind))
    args = {"q_off": 5, "kv_off": 2, "nq": 6, "nk": 10} if pin is test_zero_scale_gives_prefix_mean else {}
    with pytest.raises(AssertionError):
        pin(**args)


def test_planted_value_suffix_is_caught(monkeypatch):
    orig = mla_ref.dense_mla

    def mutant(q, kv, head_dim_v, scale, **kw):
        return orig(q, kv, head_dim_v, scale, v=np.asarray(kv)[..., -head_dim_v:], **kw)
    monkeypatch.setattr(oracle, "dense_mla", mutant)
    with pytest.raises(AssertionError):
        test_golden_dense()


def test_planted_merge_sign_is_caught(monkeypatch):
    orig = mla_ref.merge

    def mutant(oa, la, ob, lb):
        o, l = orig(oa, la, ob, lb)
        return o, l - 2 * np.log1p(np.exp(-np.abs(np.asarray(la, float) - np.asarray(lb, float))))
    monkeypatch.setattr(mla_ref, "merge", mutant)
    monkeypatch.setattr(oracle, "merge", mutant)
    with pytest.raises(AssertionError):
        test_golden_merge()


def test_planted_decode_short_by_one_is_caught(monkeypatch):
    orig = mla_ref.decode_mla

    def mutant(q, kv, kv_lens, head_dim_v, scale, kv_slots=None):
        lens = [kv.shape[1]] * q.shape[0] if kv_lens is None else list(kv_lens)
        return orig(q, kv, [max(0, int(n) - 1) for n in lens], head_dim_v, scale, kv_slots)
    monkeypatch.setattr(oracle, "decode_mla", mutant)
    with pytest.raises(AssertionError):
        test_decode_zero_scale_prefix_mean()


def test_planted_split_top_left_alignment_is_caught(monkeypatch):
    """Queries aligned to the first key instead of the last (positions
    restarting at 0 for both) must fail the chunked-prefill pin."""
    orig = mla_ref.attention

    def mutant(q, k, v, scale, causal, q_pos, k_pos):
        q_pos = np.asarray(q_pos)
        return orig(q, k, v, scale, causal, q_pos - (q_pos.min() if q_pos.size else 0), k_pos)
    monkeypatch.setattr(mla_ref, "attention", mutant)
    with pytest.raises(AssertionError):
        test_split_two_row_causal_is_chunked_prefill()
