"""Pins of the FP8 form's oracle and of its derived output tolerance.

* e4m3 decoding against torch's float8_e4m3fn (a library routine) for all
  256 codes, and against values worked out by hand from the format.
* The FP8 attention against brute force over hand-decoded values, against
  torch's scaled_dot_product_attention in float64, and against the scale
  invariant (the per-tensor scales act exactly as a score scale and a value
  scale).
* The exact weights: rows sum to one, they reproduce the output, and Z is
  exp(LSE - max).
* The tolerance (tests/fp8_bound.py): the P rounding the kernel's FP8 P.V
  product makes is emulated here with torch's e4m3 rounding, against a
  reference max anywhere in the range the kernel allows; the emulated output
  stays within the bound over random and adversarial rows, while planted
  mistakes (the dominant key dropped, the value column shifted, the value
  scale dropped) exceed it.
"""
import math

import numpy as np
import pytest
import torch

import fp8_bound
import oracle
import workloads as W
from test_oracle import brute_attention


# ------------------------------------------------------------------ decoding
def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))   # -0 at 0x80


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0), (0x3F, 1.875),
    (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x5A, 1.25 * 2.0 ** 4),
])
def test_e4m3_decode_hand_worked(code, value):
    """sign | exponent (bias 7) | 3 mantissa bits: e.g. 0x5A = 0.1011.010 =
    (1 + 2/8) * 2^(11 - 7) = 20."""
    assert oracle.e4m3_decode(np.array([code], dtype=np.uint8))[0] == value


def test_e4m3_nan_codes():
    d = oracle.e4m3_decode(np.array([0x7F, 0xFF, 0x77, 0x6F], dtype=np.uint8))
    assert np.isnan(d[0]) and np.isnan(d[1]) and d[2] == 240.0 and d[3] == 120.0


def test_workload_codes_round_trip():
    """The generator's codes decode to the e4m3 value nearest to each draw."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(4)
    d = oracle.e4m3_decode(W.to_e4m3_codes(x))
    grid = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[~np.isnan(grid)])
    nearest = np.abs(x[:, None].astype(np.float64) - grid[None, :]).min(axis=1)
    assert np.array_equal(np.abs(d - x), nearest)


# ---------------------------------------------------------------- attention
def test_fp8_attention_matches_brute_force():
    c = W.fp8_dense_case(B=1, H=2, N=6, Nkv=9, dk=12, dv=8, seed=5, q_scale=0.5, kv_scale=2.0, q_offset=3)
    out, lse = oracle.dense_mla_fp8(c.q8, c.kv8, c.q_scale, c.kv_scale, 8, 0.3, q_offset=3)
    for h in range(2):
        q = [[oracle.e4m3_decode(np.array([x], np.uint8))[0] * 0.5 for x in row] for row in c.q8[0, h]]
        k = [[oracle.e4m3_decode(np.array([x], np.uint8))[0] * 2.0 for x in row] for row in c.kv8[0, 0]]
        v = [row[:8] for row in k]
        bo, bl = brute_attention(q, k, v, 0.3, True, list(range(3, 9)), list(range(9)))
        np.testing.assert_allclose(out[0, h], bo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], bl, rtol=0, atol=1e-12)


def test_fp8_attention_matches_sdpa_float64():
    c = W.fp8_dense_case(B=1, H=3, N=40, dk=64, dv=32, seed=6)
    out, lse = oracle.dense_mla_fp8(c.q8, c.kv8, 1.0, 1.0, 32, 0.125)
    q = torch.from_numpy(oracle.e4m3_decode(c.q8))
    kv = torch.from_numpy(oracle.e4m3_decode(c.kv8)).expand(1, 3, 40, 64)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kv, kv[..., :32].contiguous(), is_causal=True,
                                                           scale=0.125)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_fp8_scales_are_a_score_scale_and_a_value_scale():
    """decode(q8) a . decode(kv8) b under scale s is decode(q8) . decode(kv8)
    under scale s a b, and the value rows carry b: O(a, b, s) = b O(1, 1, s a b)
    with the same LSE."""
    c = W.fp8_dense_case(B=1, H=2, N=30, dk=48, dv=16, seed=7)
    o1, l1 = oracle.dense_mla_fp8(c.q8, c.kv8, 0.25, 4.0, 16, 0.2)
    o2, l2 = oracle.dense_mla_fp8(c.q8, c.kv8, 1.0, 1.0, 16, 0.2 * 0.25 * 4.0)
    np.testing.assert_allclose(o1, 4.0 * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_attention_weights_consistent():
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((20, 16)), rng.standard_normal((25, 16))
    v = k[:, :8]
    qp, kp = np.arange(5, 25), np.arange(25)
    w, Z = oracle.attention_weights(q, k, 0.4, True, qp, kp)
    o, lse = oracle.attention(q, k, v, 0.4, True, qp, kp)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(w @ v, o, rtol=0, atol=1e-12)
    s = 0.4 * (q @ k.T)
    m = np.array([s[i, :qp[i] + 1].max() for i in range(20)])
    np.testing.assert_allclose(Z, np.exp(lse - m), rtol=1e-12, atol=0)
    assert (w[np.arange(20)[:, None], np.arange(25)[None, :]][kp[None, :] > qp[:, None]] == 0).all()


# ------------------------------------------------------------------ tolerance
def _e4m3_round(x):
    """Round to the nearest e4m3 value with torch (a library routine)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _emulate_fp8_pv(s_nat, v, mu_below_max):
    """The P rounding of the kernel's FP8 P.V product, for one row: weights
    2^(s - mu) (mu = the row max minus mu_below_max, in log2 units) rounded to
    e4m3, output = sum p~ v / sum p~ in fp64."""
    t = s_nat / math.log(2.0)
    mu = t.max() - mu_below_max
    p = np.exp2(t - mu)
    assert p.max() <= 256.0
    pq = _e4m3_round(p)
    return (pq @ v) / pq.sum()


def _rows(seed, n_rows, n_max, v_scale=1.0, s_scale=1.0):
    rng = np.random.default_rng(seed)
    for _ in range(n_rows):
        n = int(rng.integers(1, n_max + 1))
        s = rng.standard_normal(n) * math.sqrt(3.0) * s_scale
        v = rng.standard_normal((n, 16)) * v_scale
        yield rng, s, v


def _exact(s, v):
    e = np.exp(s - s.max())
    Z = e.sum()
    w = e / Z
    return w, Z, w @ v


@pytest.mark.parametrize("seed,n_max,v_scale,s_scale", [
    (20, 8, 1.0, 1.0),        # few keys
    (21, 3000, 1.0, 1.0),     # long rows, the score spread of the workloads
    (22, 40, 4.0, 3.0),       # large values, sharp weights
    (23, 2000, 1.0, 0.1),     # nearly uniform weights: most of them in the e4m3 normal range
])
def test_emulated_fp8_pv_stays_within_bound(seed, n_max, v_scale, s_scale):
    worst = 0.0
    for rng, s, v in _rows(seed, 60, n_max, v_scale, s_scale):
        w, Z, o = _exact(s, v)
        for below in (0.0, float(rng.uniform(0, 8)), 8.0):
            got = _emulate_fp8_pv(s, v, below)
            b = fp8_bound.o_bound(w[None], np.array([Z]), v, o[None], bf16=False)[0]
            worst = max(worst, float((np.abs(got - o) / b).max()))
    print(f"worst emulated error / bound: {worst:.3f}")
    assert worst <= 1.0


def test_fp8_bound_catches_planted_mistakes():
    """On rows of 2..60 keys, three mistakes each exceed the bound on some
    element: the dominant key dropped, the value columns shifted by one, the
    value scale dropped (values 4x too small)."""
    caught = {"drop": 0, "shift": 0, "scale": 0}
    n = 0
    for rng, s, v in _rows(30, 40, 60, 1.0, 1.0):
        if len(s) < 2:
            continue
        n += 1
        w, Z, o = _exact(s, v)
        b = fp8_bound.o_bound(w[None], np.array([Z]), v, o[None], bf16=True)[0]
        keep = np.arange(len(s)) != int(np.argmax(s))
        wd = np.exp(s[keep] - s[keep].max())
        caught["drop"] += bool((np.abs((wd / wd.sum()) @ v[keep] - o) > b).any())
        caught["shift"] += bool((np.abs(np.roll(o, 1) - o) > b).any())
        caught["scale"] += bool((np.abs(o / 4.0 - o) > b).any())
    print(caught, "of", n)
    assert all(c == n for c in caught.values()), caught
