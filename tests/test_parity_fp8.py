"""Parity of the FP8 form (mla_fwd_fp8, through the C ABI) with the fp64
oracle: the attention of the dequantised e4m3 inputs.

The output is held to the bound derived from the kernel's e4m3 P
(tests/fp8_bound.py), the LSE to max-abs 1e-3, and every case also checks
that no NaN appears and that rows without a visible key give (0, -inf).
Where the rounding of P is exact (scale 0: every weight is 1), the output is
held to the bf16 form's bound (1e-2 below |O| = 2).
"""
import numpy as np
import pytest

import fp8_bound
import oracle
import workloads as W
from gpu_util import LSE_TOL, dev, host, report, report_o

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mla():
    import ring_chunk_attention_amd as m
    return m


def _codes(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().view(torch.float8_e4m3fn)


def _gpu(mla, c, **kw):
    out, lse = mla.fwd_fp8(_codes(c.q8), _codes(c.kv8), scale=c.scale, q_scale=c.q_scale, kv_scale=c.kv_scale,
                           causal=c.causal, q_offset=c.q_offset, kv_offset=c.kv_offset, **kw)
    torch.cuda.synchronize()
    return out, lse


def _ref(c, rows=None, heads=None):
    """(O, LSE, bound) of the oracle for the given rows / heads (the heads are
    sliced out of the codes first, so that only they are decoded)."""
    B, H, N = c.q8.shape[:3]
    Nkv = c.kv8.shape[2]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    heads = np.arange(H) if heads is None else np.asarray(heads)
    q8 = c.q8[:, heads]
    o, l = oracle.dense_mla_fp8(q8, c.kv8, c.q_scale, c.kv_scale, 512, c.scale, causal=c.causal,
                                q_offset=c.q_offset, kv_offset=c.kv_offset, rows=rows)
    kv = oracle.e4m3_decode(c.kv8) * c.kv_scale
    bound = np.empty_like(o)
    for b in range(B):
        for hi in range(len(heads)):
            q = oracle.e4m3_decode(q8[b, hi, rows]) * c.q_scale
            w, Z = oracle.attention_weights(q, kv[b, 0], c.scale, c.causal, c.q_offset + rows,
                                            c.kv_offset + np.arange(Nkv))
            bound[b, hi] = fp8_bound.o_bound(w, Z, kv[b, 0, :, :512], o[b, hi])
    return o, l, bound


def _check(name, out, lse, o_ref, l_ref, bound):
    got = host(out)
    assert fp8_bound.check(f"{name} O", got, o_ref, bound) <= 1.0
    assert report(f"{name} LSE", host(lse), l_ref) <= LSE_TOL


def test_fp8_tiny_full(mla):
    """4 heads x 128 causal rows, every element."""
    c = W.fp8_dense_case(B=1, H=4, N=128, seed=0)
    out, lse = _gpu(mla, c)
    _check("fp8 tiny", out, lse, *_ref(c))


@pytest.mark.parametrize("B,H,N,Nkv,q_off,kv_off,causal,qs,ks,seed", [
    (2, 6, 200, 200, 0, 0, True, 1.0, 1.0, 1),          # ragged rows and heads, two batches
    (1, 5, 77, 150, 73, 0, True, 1.0, 1.0, 2),          # queries at the end of a longer key range
    (1, 4, 64, 96, 0, 40, True, 1.0, 1.0, 3),           # keys start later: first rows see nothing
    (1, 3, 45, 70, 0, 0, False, 1.0, 1.0, 4),           # no mask, ragged key tail
    (1, 8, 1, 300, 299, 0, True, 1.0, 1.0, 5),          # a single query row
    (1, 4, 130, 130, 0, 0, True, 0.5, 2.0, 6),          # non-unit scales
    (1, 7, 100, 513, 413, 0, True, 0.125, 0.25, 7),     # scales and a 64-key tile boundary crossing
])
def test_fp8_ragged(mla, B, H, N, Nkv, q_off, kv_off, causal, qs, ks, seed):
    c = W.fp8_dense_case(B=B, H=H, N=N, Nkv=Nkv, seed=seed, q_scale=qs, kv_scale=ks, causal=causal,
                         q_offset=q_off, kv_offset=kv_off)
    out, lse = _gpu(mla, c)
    _check("fp8 ragged", out, lse, *_ref(c))


def test_fp8_zero_scale_is_the_prefix_mean(mla):
    """scale 0: every visible weight is exactly 1 (also in e4m3), so O is the
    mean of the visible value rows and LSE = ln(#visible); held to the bf16
    bound, which checks the value operand's layout exactly."""
    c = W.fp8_dense_case(B=1, H=4, N=150, Nkv=170, seed=8, q_offset=20, scale=0.0)
    out, lse = _gpu(mla, c)
    o_ref, l_ref = oracle.dense_mla_fp8(c.q8, c.kv8, 1.0, 1.0, 512, 0.0, q_offset=20)
    assert report_o("fp8 scale 0 O", host(out), o_ref) <= 1.0
    assert report("fp8 scale 0 LSE", host(lse), l_ref) <= LSE_TOL


def test_fp8_wide_range_second_pass(mla):
    """Softmax scale 8/sqrt(192): scores of about 14 nats standard deviation,
    so row maxima grow past the first tile's by far more than 8 log2 units
    and the workgroups take the exact-max second pass."""
    c = W.fp8_dense_case(B=1, H=4, N=300, seed=9, scale=8.0 * W.SCALE_192)
    q = oracle.e4m3_decode(c.q8[0, 0])
    k = oracle.e4m3_decode(c.kv8[0, 0])
    s = (q @ k.T) * c.scale / np.log(2.0)
    s = np.where(np.tril(np.ones((300, 300), dtype=bool)), s, -np.inf)
    growth = (s.max(axis=1) - np.array([row[:min(64, i + 1)].max() for i, row in enumerate(s)]))
    assert growth.max() > 8.0
    out, lse = _gpu(mla, c)
    _check("fp8 wide", out, lse, *_ref(c))


def test_fp8_large_products(mla):
    """RoPE columns of q and kv times 8 (exact in e4m3): single products
    reach ~1e3, where the 8-bit MFMA's block sums lose low bits; the LSE is
    held to the bound derived from that resolution (tests/fp8_bound.py), O to
    the P bound."""
    c = W.fp8_dense_case(B=1, H=4, N=300, seed=9)
    for t in (c.q8, c.kv8):
        d = oracle.e4m3_decode(t[..., 512:]) * 8.0
        assert np.abs(d).max() <= 448
        t[..., 512:] = W.to_e4m3_codes(d.astype(np.float32))
    out, lse = _gpu(mla, c)
    o_ref, l_ref, bound = _ref(c)
    assert fp8_bound.check("fp8 large products O", host(out), o_ref, bound) <= 1.0
    q = oracle.e4m3_decode(c.q8[0])
    k = oracle.e4m3_decode(c.kv8[0, 0])
    vis = np.tril(np.ones((300, 300), dtype=bool))
    lb = np.stack([fp8_bound.lse_bound(q[h], k, c.scale, vis) for h in range(4)])[None]
    err = np.abs(host(lse) - l_ref)
    print(f"fp8 large products LSE: max err {err.max():.3e}, worst against its bound {(err / lb).max():.3f}")
    assert (err <= lb).all()


def test_fp8_empty_rows_and_sizes(mla):
    c = W.fp8_dense_case(B=1, H=4, N=40, Nkv=64, seed=10)
    q8, kv8 = _codes(c.q8), _codes(c.kv8)
    z = torch.empty((1, 1, 0, 576), dtype=torch.uint8, device="cuda")
    out, lse = mla.fwd_fp8(q8, z, scale=c.scale)                     # no key rows
    torch.cuda.synchronize()
    assert (host(out) == 0).all() and np.isneginf(host(lse)).all()
    out, lse = mla.fwd_fp8(torch.empty((1, 4, 0, 576), dtype=torch.uint8, device="cuda"), kv8, scale=c.scale)
    assert out.shape == (1, 4, 0, 512)


def test_fp8_queue_bit_identical_and_deterministic(mla):
    """B = 2, 32 heads, N = 2048: enough row blocks for the item queue; with
    and without the workspace, and twice, the same bits."""
    c = W.fp8_dense_case(B=2, H=32, N=2048, seed=11)
    q8, kv8 = _codes(c.q8), _codes(c.kv8)
    o1, l1 = mla.fwd_fp8(q8, kv8, scale=c.scale, workspace=None)
    o2, l2 = mla.fwd_fp8(q8, kv8, scale=c.scale)
    o3, l3 = mla.fwd_fp8(q8, kv8, scale=c.scale)
    torch.cuda.synchronize()
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o.view(torch.int16), o1.view(torch.int16)) and torch.equal(l, l1)
    rows, heads = [0, 1, 63, 64, 1000, 2047], [0, 31]
    o_ref, l_ref, bound = _ref(W.Fp8DenseCase(c.q8[1:], c.kv8[1:], 1.0, 1.0, 512, c.scale), rows=rows, heads=heads)
    got_o = o1[1:][:, heads][:, :, rows]
    got_l = l1[1:][:, heads][:, :, rows]
    _check("fp8 queue", got_o, got_l, o_ref, l_ref, bound)


def test_fp8_dsv3_full_size_sampled(mla):
    """128 heads x 8192 causal rows in e4m3 (the benchmarked launch):
    sampled rows of four heads against the oracle, plus whole-output
    sanity."""
    c = W.dsv3_prefill_fp8(0)
    out, lse = _gpu(mla, c)
    heads = [0, 37, 90, 127]
    rows = np.unique(np.concatenate([[0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 4095, 4096, 8190, 8191],
                                     np.random.default_rng(1).integers(0, 8192, 34)]))
    o_ref, l_ref, bound = _ref(c, rows=rows, heads=heads)
    _check("fp8 dsv3", out[:, heads][:, :, rows], lse[:, heads][:, :, rows], o_ref, l_ref, bound)
    assert not torch.isnan(out).any() and torch.isfinite(lse).all()


@pytest.mark.parametrize("N,q_off", [(100, 0), (40, 37), (7, 0)])
def test_fp8_unseen_key_rows_do_not_reach_the_output(mla, N, q_off):
    """As for the bf16 form: key rows past the last query's position hold
    e4m3 NaN codes (0x7f) from the first unseen row on, inside the last
    visible tile and after it; the outputs equal the call on the clean rows
    bitwise and hold no NaN."""
    c = W.fp8_dense_case(B=1, H=4, N=N, Nkv=300, seed=71, q_offset=q_off)
    dirty = c.kv8.copy()
    dirty[:, :, q_off + N:, :] = 0x7F
    a, la = mla.fwd_fp8(_codes(c.q8), _codes(c.kv8), scale=c.scale, q_offset=q_off)
    b, lb = mla.fwd_fp8(_codes(c.q8), _codes(dirty), scale=c.scale, q_offset=q_off)
    torch.cuda.synchronize()
    assert not torch.isnan(b).any() and not torch.isnan(lb).any()
    assert torch.equal(a, b) and torch.equal(la, lb)
