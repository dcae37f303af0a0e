"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case draws seeded inputs from ``workloads``, runs them through
``ring_chunk_attention_amd`` on the GPU and compares element by element with
the oracle: bf16 outputs to 1e-2 max-abs where |O| < 2 and, from |O| = 2
on, to half an ulp plus 1e-2 (the rounding of a value within 1e-2), fp32 LSE
to 1e-3 max-abs; gathers and the repeated-row case bit-exact.  Cases whose outputs
reach |O| >= 2 (folds with a previous result, wide score ranges, rows that
see few keys) also run with a float32 output: that result, the kernel's
arithmetic before the last rounding, must lie within 1e-2 of the oracle
everywhere, and the bf16 result must be bit for bit its round-to-nearest-even.
Small cases compare every element; the full-size workloads (the launch
configurations the benchmark times) compare sampled rows that the oracle
computes one by one.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import LSE_TOL, O_TOL, assert_rne_of, dev, dev_bf16, host, report, report_o

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mla():
    import ring_chunk_attention_amd as m
    return m


def _twin(name, o_bf16, o_f32, o_ref, got_bf16=None, got_f32=None):
    """A call's bf16 and float32 outputs against the oracle: the float32 one
    within max-abs 1e-2 everywhere, the bf16 one its rounding bit for bit and
    within the bf16 bound.  got_*: the host values to compare with o_ref (the
    sampled rows), when not the whole tensors."""
    assert_rne_of(name, o_bf16, o_f32)
    g16 = host(o_bf16) if got_bf16 is None else got_bf16
    g32 = host(o_f32) if got_f32 is None else got_f32
    assert report(f"{name} fp32 O", g32, o_ref) <= O_TOL
    assert report_o(f"{name} O", g16, o_ref) <= 1.0


def _f32(t):
    return torch.empty(t.shape, dtype=torch.float32, device=t.device)


# ---------------------------------------------------------------------------
# shared-latent dense
# ---------------------------------------------------------------------------
def _dense_gpu(mla, c, **kw):
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    out, lse = mla.fwd(q, kv, scale=c.scale, head_dim_v=c.head_dim_v, causal=c.causal,
                       q_offset=c.q_offset, kv_offset=c.kv_offset, **kw)
    torch.cuda.synchronize()
    return out, lse


def test_tiny_config_full(mla):
    """B=1, 4 heads, N=128, dk=576/dv=512, seed 0: every element, with the
    float32-output twin (early rows see few keys and reach |O| > 2)."""
    c = W.tiny(0)
    out, lse = _dense_gpu(mla, c)
    o32, l32 = _dense_gpu(mla, c, out=_f32(out))
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    _twin("tiny", out, o32, o_ref)
    assert report("tiny LSE", host(lse), l_ref) <= LSE_TOL
    assert torch.equal(lse, l32)


@pytest.mark.parametrize("B,H,N,Nkv,q_off,kv_off,causal,seed", [
    (2, 6, 200, 200, 0, 0, True, 1),       # ragged rows and heads, two batches
    (1, 5, 77, 150, 73, 0, True, 2),       # queries at the end of a longer key range
    (1, 4, 64, 96, 0, 40, True, 3),        # keys start later: first rows see nothing
    (1, 3, 45, 70, 0, 0, False, 4),        # no mask, ragged key tail
    (1, 8, 1, 300, 299, 0, True, 5),       # a single query row (decode-like)
])
def test_dense_ragged(mla, B, H, N, Nkv, q_off, kv_off, causal, seed):
    c = W.dense_case(B=B, H=H, N=N, Nkv=Nkv, seed=seed, causal=causal, q_offset=q_off,
                     kv_offset=kv_off)
    out, lse = _dense_gpu(mla, c)
    o32, _ = _dense_gpu(mla, c, out=_f32(out))
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale, causal=causal, q_offset=q_off,
                                    kv_offset=kv_off)
    _twin("ragged", out, o32, o_ref)
    assert report("LSE", host(lse), l_ref) <= LSE_TOL


@pytest.mark.parametrize("N,q_off", [(100, 0), (100, 37), (40, 0), (40, 37), (7, 0)])
def test_unseen_key_rows_do_not_reach_the_output(mla, N, q_off):
    """Key rows that no query of the call can see (causal, past the last
    query's position) are never part of the result, whatever they hold: NaN
    there (bf16 0x7fc0), in the rows right after the last visible one inside
    its tile and in every later tile, leaves the outputs equal to the call on
    the clean rows (bitwise) and to the oracle.  With N = 40 and 7 the last
    visible key falls in one of the first three key tiles, which the key loop
    copies before it starts."""
    Nkv = 300
    c = W.dense_case(B=1, H=4, N=N, Nkv=Nkv, seed=41, q_offset=q_off)
    first_unseen = q_off + N  # the last query sits at q_off + N - 1
    dirty = c.kv.copy()
    dirty[:, :, first_unseen:, :] = 0x7fc0
    q = dev_bf16(c.q)
    a, la = mla.fwd(q, dev_bf16(c.kv), scale=c.scale, q_offset=q_off)
    b, lb = mla.fwd(q, dev_bf16(dirty), scale=c.scale, q_offset=q_off)
    torch.cuda.synchronize()
    assert not torch.isnan(b).any() and not torch.isnan(lb).any()
    assert torch.equal(a, b) and torch.equal(la, lb)
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale, q_offset=q_off)
    assert report_o("unseen rows O", host(b), o_ref) <= 1.0
    assert report("unseen rows LSE", host(lb), l_ref) <= LSE_TOL


def test_dense_rope_split_equals_single_tensor(mla):
    """Passing the 64 RoPE columns as separate q_rope/k_rope tensors reads the
    same values: bitwise equal to the single 576-column call."""
    c = W.dense_case(B=1, H=4, N=100, seed=6)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    a, la = mla.fwd(q, kv, scale=c.scale)
    qa, qr = q[..., :512].contiguous(), q[..., 512:].contiguous()
    ka, kr = kv[..., :512].contiguous(), kv[..., 512:].contiguous()
    b, lb = mla.fwd(qa, ka, q_rope=qr, k_rope=kr, scale=c.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_dense_fold_prev(mla):
    """prev_out/prev_lse folded in the epilogue equals the oracle merge of the
    previous pair with the fresh result; rows with prev_lse = -inf keep the
    fresh result, rows without visible keys keep prev exactly."""
    c = W.dense_case(B=1, H=4, N=96, Nkv=96, seed=7, q_offset=0, kv_offset=32)
    rng = np.random.default_rng(70)
    prev_o = W.normal_bf16(rng, (1, 4, 96, 512))
    prev_l = rng.uniform(0, 8, (1, 4, 96)).astype(np.float32)
    prev_l[:, :, 5] = -np.inf
    out, lse = _dense_gpu(mla, c, prev=(dev_bf16(prev_o), dev(prev_l)))
    o32, l32 = _dense_gpu(mla, c, prev=(dev_bf16(prev_o), dev(prev_l)), out=_f32(out))
    fresh = oracle.dense_mla(c.q, c.kv, 512, c.scale, q_offset=0, kv_offset=32)
    o_ref, l_ref = oracle.merge(prev_o, prev_l, fresh[0], fresh[1])
    _twin("fold", out, o32, o_ref)
    assert report("fold LSE", host(lse), l_ref) <= LSE_TOL
    assert torch.equal(lse, l32)
    # rows 0..31 see no key (kv starts at 32): the previous values are kept bit
    # for bit, except row 5 whose previous LSE is -inf too, which gives (0, -inf)
    keep = [i for i in range(32) if i != 5]
    got = out[:, :, keep].view(torch.int16).cpu().numpy()
    assert np.array_equal(got, prev_o[:, :, keep].view(np.int16))
    assert torch.all(out[:, :, 5] == 0) and torch.all(torch.isneginf(lse[:, :, 5]))


def test_dense_fold_in_place(mla):
    c = W.dense_case(B=1, H=4, N=64, seed=8)
    rng = np.random.default_rng(80)
    prev_o = W.normal_bf16(rng, (1, 4, 64, 512))
    prev_l = rng.uniform(0, 8, (1, 4, 64)).astype(np.float32)
    o_t, l_t = dev_bf16(prev_o), dev(prev_l)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    mla.fwd(q, kv, scale=c.scale, prev=(o_t, l_t), out=o_t, lse=l_t)
    # the float32 twin, in place over a float32 copy of the same previous result
    o_f, l_f = dev_bf16(prev_o).float(), dev(prev_l)
    mla.fwd(q, kv, scale=c.scale, prev=(o_f, l_f), out=o_f, lse=l_f)
    torch.cuda.synchronize()
    fresh = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    o_ref, l_ref = oracle.merge(prev_o, prev_l, fresh[0], fresh[1])
    _twin("in-place", o_t, o_f, o_ref)
    assert report("in-place LSE", host(l_t), l_ref) <= LSE_TOL
    assert torch.equal(l_t, l_f)


def test_dense_fp32_out_and_prev(mla):
    """float32 out and prev_out (the ring carry): the output skips the final
    bf16 rounding, so this bounds the kernel's own arithmetic error."""
    c = W.dense_case(B=1, H=8, N=160, seed=10)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    out = torch.empty((1, 8, 160, 512), dtype=torch.float32, device="cuda")
    _, lse = mla.fwd(q, kv, scale=c.scale, out=out)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    err = report("fp32 out O", host(out), o_ref)
    assert err <= O_TOL
    assert report("fp32 out LSE", host(lse), l_ref) <= LSE_TOL
    # fold into a float32 previous result, writing bf16
    rng = np.random.default_rng(100)
    prev_o = rng.standard_normal((1, 8, 160, 512)).astype(np.float32)
    prev_l = rng.uniform(0, 8, (1, 8, 160)).astype(np.float32)
    o2, l2 = mla.fwd(q, kv, scale=c.scale, prev=(dev(prev_o), dev(prev_l)))
    torch.cuda.synchronize()
    m_o, m_l = oracle.merge(prev_o, prev_l, o_ref, l_ref)
    assert report_o("fp32 prev O", host(o2), m_o) <= 1.0
    assert report("fp32 prev LSE", host(l2), m_l) <= LSE_TOL


def test_dense_deterministic(mla):
    c = W.dense_case(B=1, H=8, N=256, seed=9)
    a = _dense_gpu(mla, c)
    b = _dense_gpu(mla, c)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_dsv3_full_size_sampled(mla):
    """128 heads x 8192 causal rows (the benchmark's launch): sampled rows of
    four heads against the oracle, plus whole-output sanity."""
    c = W.dsv3_prefill(0)
    out, lse = _dense_gpu(mla, c)
    heads = [0, 37, 90, 127]
    rows = np.unique(np.concatenate([[0, 1, 2, 31, 32, 33, 127, 128, 4095, 4096, 8190, 8191],
                                     np.random.default_rng(1).integers(0, 8192, 52)]))
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale, rows=rows, heads=heads)
    o_got = host(out[:, heads][:, :, rows])
    l_got = host(lse[:, heads][:, :, rows])
    assert report_o("dsv3 O", o_got, o_ref) <= 1.0
    assert report("dsv3 LSE", l_got, l_ref) <= LSE_TOL
    assert not torch.isnan(out).any() and torch.isfinite(lse).all()
    # the float32 twin: the whole output is its rounding, the sampled rows within 1e-2
    o32, l32 = _dense_gpu(mla, c, out=_f32(out))
    assert torch.equal(lse, l32)
    assert_rne_of("dsv3", out, o32)
    assert report("dsv3 fp32 O", host(o32[:, heads][:, :, rows]), o_ref) <= O_TOL


# ---------------------------------------------------------------------------
# merge and one-device ring
# ---------------------------------------------------------------------------
def test_merge_kernel(mla):
    rng = np.random.default_rng(20)
    oa = W.normal_bf16(rng, (2, 3, 50, 512))
    ob = W.normal_bf16(rng, (2, 3, 50, 512))
    la = rng.uniform(-5, 5, (2, 3, 50)).astype(np.float32)
    lb = rng.uniform(-5, 5, (2, 3, 50)).astype(np.float32)
    la[0, 0, :3] = -np.inf
    lb[0, 0, 2:5] = -np.inf
    out, lse = mla.merge(dev_bf16(oa), dev(la), dev_bf16(ob), dev(lb))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge(oa, la, ob, lb)
    assert report_o("merge O", host(out), o_ref) <= 1.0
    assert report("merge LSE", host(lse), l_ref) <= LSE_TOL


def test_merge_in_place_dv128(mla):
    rng = np.random.default_rng(21)
    oa = W.normal_bf16(rng, (1, 4, 33, 128))
    ob = W.normal_bf16(rng, (1, 4, 33, 128))
    la = rng.uniform(-5, 5, (1, 4, 33)).astype(np.float32)
    lb = rng.uniform(-5, 5, (1, 4, 33)).astype(np.float32)
    ta, tl = dev_bf16(oa), dev(la)
    mla.merge(ta, tl, dev_bf16(ob), dev(lb), out=ta, lse=tl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge(oa, la, ob, lb)
    assert report_o("merge in place O", host(ta), o_ref) <= 1.0
    assert report("merge in place LSE", host(tl), l_ref) <= LSE_TOL


def test_merge_wide_rows_nan_side_and_empty_rows(mla):
    """dv = 1024 (columns past the first 512), a ragged row count, the output
    written in place over the b side, a side of LSE -inf whose rows hold NaN
    (weight 0: never multiplied) and rows with both sides -inf (O = 0,
    LSE = -inf)."""
    rng = np.random.default_rng(22)
    oa = W.normal_bf16(rng, (1, 1, 37, 1024))
    ob = W.normal_bf16(rng, (1, 1, 37, 1024))
    la = rng.uniform(-5, 5, (1, 1, 37)).astype(np.float32)
    lb = rng.uniform(-5, 5, (1, 1, 37)).astype(np.float32)
    la[0, 0, 5:9] = -np.inf
    oa[0, 0, 5:9] = 0x7fc0                        # bf16 NaN rows on the side of weight 0
    lb[0, 0, 7:12] = -np.inf
    ob[0, 0, 10:12] = 0x7fc0
    tb, tl = dev_bf16(ob), dev(lb)
    mla.merge(dev_bf16(oa), dev(la), tb, tl, out=tb, lse=tl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge(oa, la, ob, lb)   # the oracle multiplies no weight-0 side either
    got_o, got_l = host(tb), host(tl)
    assert not np.isnan(got_o).any()
    assert (got_o[0, 0, 7:9] == 0).all() and np.isneginf(got_l[0, 0, 7:9]).all()
    assert report_o("merge wide O", got_o, o_ref) <= 1.0
    assert report("merge wide LSE", got_l, l_ref) <= LSE_TOL


@pytest.mark.parametrize("order", ["ring", "balanced"])
@pytest.mark.parametrize("H,N,P", [(4, 256, 4), (3, 192, 3), (2, 96, 1), (2, 640, 5),
                                   (2, 512, 8),       # 8 diagonals: two group launches
                                   (2, 2048, 64),     # the most chunks: 2080 calls in 64 launches
                                   (3, 250, 4),       # ragged: chunks of 63, the last 61
                                   (2, 129, 8)])      # ragged: chunks of 17, the last 10
def test_ring_small_equals_unchunked_oracle(mla, H, N, P, order):
    c = W.dense_case(B=1, H=H, N=N, seed=30 + P)
    out, lse = mla.ring_fwd(dev_bf16(c.q), dev_bf16(c.kv), P, scale=c.scale, order=order)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    assert report_o("ring O", host(out), o_ref) <= 1.0
    assert report("ring LSE", host(lse), l_ref) <= LSE_TOL


@pytest.mark.parametrize("order", ["ring", "balanced"])
def test_ring4_config_sampled(mla, order):
    """16 heads, N = 4096 in 4 chunks of 1024, in ring order and in the
    balanced schedule: sampled rows of four heads against the unchunked
    oracle."""
    c = W.ring4(0)
    out, lse = mla.ring_fwd(dev_bf16(c.q), dev_bf16(c.kv), 4, scale=c.scale, order=order)
    torch.cuda.synchronize()
    heads = [0, 5, 10, 15]
    rows = np.array([0, 1, 511, 1023, 1024, 1025, 2047, 2048, 3071, 3072, 3073, 4094, 4095])
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale, rows=rows, heads=heads)
    assert report_o("ring4 O", host(out[:, heads][:, :, rows]), o_ref) <= 1.0
    assert report("ring4 LSE", host(lse[:, heads][:, :, rows]), l_ref) <= LSE_TOL


@pytest.mark.parametrize("order", ["ring", "balanced"])
@pytest.mark.parametrize("B,H,N,P", [(1, 8, 640, 5), (2, 4, 250, 4), (1, 4, 70, 8), (1, 2, 10, 8)])
def test_ring_bit_identical_to_its_calls(mla, order, B, H, N, P):
    """The ring's single launch runs, for each query chunk, the calls the
    pages describe: the same bits as those calls made one by one through
    mla_fwd in the chunk's fold order (the schedule's step order), with a
    float32 running result between them and the bf16 output from the last.
    Ragged and empty chunks included (N = 70 in 8 chunks of 9: the last one
    has 7 rows; N = 10 in 8 chunks of 2: the last three are empty)."""
    c = W.dense_case(B=B, H=H, N=N, seed=90 + P)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    out, lse = mla.ring_fwd(q, kv, P, scale=c.scale, order=order)
    step_of = {rk: s for s, calls in enumerate(mla.ring_schedule(P, order)) for rk in calls}
    C = -(-N // P)
    ref_o, ref_l = torch.empty_like(out), torch.empty_like(lse)
    for r in range(P):
        r0, r1 = r * C, min((r + 1) * C, N)
        if r1 <= r0:
            continue
        carry = torch.empty((B, H, r1 - r0, 512), dtype=torch.float32, device="cuda")
        lse_r = torch.empty((B, H, r1 - r0), dtype=torch.float32, device="cuda")
        for s, k in enumerate(sorted(range(r + 1), key=lambda k: step_of[(r, k)])):
            k0, k1 = k * C, min((k + 1) * C, N)
            o_r = ref_o[:, :, r0:r1] if s == r else carry
            mla.fwd(q[:, :, r0:r1], kv[:, :, k0:k1], scale=c.scale, causal=True, q_offset=r0, kv_offset=k0,
                    prev=None if s == 0 else (carry, lse_r), out=o_r, lse=lse_r, workspace=None)
        ref_l[:, :, r0:r1] = lse_r
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse, ref_l)


# ---------------------------------------------------------------------------
# split q/k varlen ring step
# ---------------------------------------------------------------------------
def _split_gpu(mla, c, with_prev=True, f32=False, causal=True, scale=None):
    args = [dev_bf16(x) for x in (c.q1, c.q2, c.k1, c.k2, c.v)]
    prev = (dev_bf16(c.prev_out), dev(c.prev_lse)) if (with_prev and c.prev_out is not None) else None
    T, H = c.q1.shape[:2]
    out = torch.empty((T, H, c.v.shape[2]), dtype=torch.float32, device="cuda") if f32 else None
    out, lse = mla.split_fwd(*args, scale=c.scale if scale is None else scale, seq_lens=dev(c.seq_lens),
                             prev=prev, out=out, causal=causal)
    torch.cuda.synchronize()
    return out, lse


def _split_twin(mla, c, with_prev=True, **kw):
    """The bf16 and float32 outputs of the same split call (same LSE)."""
    out, lse = _split_gpu(mla, c, with_prev, **kw)
    o32, l32 = _split_gpu(mla, c, with_prev, f32=True, **kw)
    assert torch.equal(lse, l32)
    return out, o32, lse


@pytest.mark.parametrize("lens,H,Hkv,with_prev", [
    ([5, 130, 1, 257, 64], 4, 2, True),
    ([300, 200], 2, 2, False),
    ([129], 3, 1, True),
])
def test_split_small(mla, lens, H, Hkv, with_prev):
    c = W.split_case(seq_lens=lens, H=H, Hkv=Hkv, seed=sum(lens), with_prev=with_prev)
    out, o32, lse = _split_twin(mla, c, with_prev)
    o_ref, l_ref = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale,
                                    prev_out=c.prev_out if with_prev else None,
                                    prev_lse=c.prev_lse if with_prev else None)
    _twin("split", out, o32, o_ref)
    assert report("split LSE", host(lse), l_ref) <= LSE_TOL


@pytest.mark.parametrize("with_prev", [False, True])
def test_split_non_causal(mla, with_prev):
    """Without the mask every token of a sequence sees every key of its own
    sequence (and none of the others)."""
    c = W.split_case(seq_lens=[70, 200, 1, 130], H=4, Hkv=2, seed=77, with_prev=with_prev)
    out, o32, lse = _split_twin(mla, c, with_prev, causal=False)
    o_ref, l_ref = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale, causal=False,
                                    prev_out=c.prev_out if with_prev else None,
                                    prev_lse=c.prev_lse if with_prev else None)
    _twin("split non-causal", out, o32, o_ref)
    assert report("split non-causal LSE", host(lse), l_ref) <= LSE_TOL


@pytest.mark.parametrize("B,Hq,Hkv,N,Nkv,q_off,kv_off,causal,with_prev", [
    (2, 4, 2, 150, 170, 20, 0, True, False),
    (1, 8, 1, 40, 300, 0, 0, True, True),       # most key rows past every query
    (2, 2, 2, 200, 90, 0, 50, False, True),     # no mask
    (1, 4, 4, 33, 33, 0, 0, True, False),
])
def test_split_form_batched_with_offsets(mla, B, Hq, Hkv, N, Nkv, q_off, kv_off, causal, with_prev):
    """The split form through mla_fwd without seq_lens: [B, H, N, D] views
    with separate nope/RoPE parts and V, query and key offsets and the mask,
    as the plain attention of the concatenated parts.  Key and value rows past
    every query's position hold NaN, which must not reach the result."""
    rng = np.random.default_rng(500 + N)
    q1, q2 = W.normal_bf16(rng, (B, Hq, N, 128)), W.normal_bf16(rng, (B, Hq, N, 64))
    k1, k2 = W.normal_bf16(rng, (B, Hkv, Nkv, 128)), W.normal_bf16(rng, (B, Hkv, Nkv, 64))
    v = W.normal_bf16(rng, (B, Hkv, Nkv, 128))
    scale = W.SCALE_192
    prev = None
    if with_prev:
        prev_o = W.normal_bf16(rng, (B, Hq, N, 128))
        prev_l = rng.uniform(0, 8, (B, Hq, N)).astype(np.float32)
    dirty = [x.copy() for x in (k1, k2, v)]
    first_unseen = q_off + N - kv_off  # key index of the first row no query sees
    if causal and first_unseen < Nkv:
        for x in dirty:
            x[:, :, max(first_unseen, 0):] = 0x7fc0

    def run(ks, f32=False):
        pv = (dev_bf16(prev_o), dev(prev_l)) if with_prev else None
        out = torch.empty((B, Hq, N, 128), dtype=torch.float32, device="cuda") if f32 else None
        o, l = mla.fwd(dev_bf16(q1), dev_bf16(ks[0]), scale=scale, causal=causal, q_offset=q_off,
                       kv_offset=kv_off, q_rope=dev_bf16(q2), k_rope=dev_bf16(ks[1]), v=dev_bf16(ks[2]),
                       prev=pv, out=out)
        torch.cuda.synchronize()
        return o, l

    out, lse = run((k1, k2, v))
    o32, l32 = run((k1, k2, v), f32=True)
    od, ld = run(dirty)
    assert torch.equal(lse, l32)
    assert not torch.isnan(od).any() and torch.equal(od, out) and torch.equal(ld, lse)
    cat = lambda a, b: np.concatenate([a, b], axis=-1)
    o_ref, l_ref = oracle.dense_mla(cat(q1, q2), cat(k1, k2), 128, scale, causal=causal, q_offset=q_off,
                                    kv_offset=kv_off, v=v)
    if with_prev:
        o_ref, l_ref = oracle.merge(prev_o, prev_l, o_ref, l_ref)
    _twin("split batched", out, o32, o_ref)
    assert report("split batched LSE", host(lse), l_ref) <= LSE_TOL


@pytest.mark.parametrize("gpu_lens,eff_lens", [
    ([50, -3, 40], [50, 40]),    # a negative length counts as 0; tokens past the sum stay unwritten
    ([100, 60], [100, 20]),      # the lengths are clipped to the tokens there are
    ([0, 70, 0], [70]),          # empty sequences around one
])
def test_split_lengths_read_on_the_device(mla, gpu_lens, eff_lens):
    """seq_lens is read on the device, unchecked before launch: a negative
    length counts as 0, the sum is clipped to T, and tokens past it keep what
    the output held."""
    T = 120
    c = W.split_case(seq_lens=eff_lens + ([T - sum(eff_lens)] if sum(eff_lens) < T else []), H=4, Hkv=2,
                     seed=93, with_prev=False)
    args = [dev_bf16(x) for x in (c.q1, c.q2, c.k1, c.k2, c.v)]
    out = torch.full((T, 4, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((4, T), 7.0, dtype=torch.float32, device="cuda")
    mla.split_fwd(*args, scale=c.scale, seq_lens=dev(np.array(gpu_lens, np.int32)), out=out, lse=lse)
    torch.cuda.synchronize()
    n = sum(eff_lens)
    o_ref, l_ref = oracle.split_mla(c.q1[:n], c.q2[:n], c.k1[:n], c.k2[:n], c.v[:n],
                                    np.array(eff_lens, np.int32), c.scale)
    o, l = host(out), host(lse)
    assert report_o("split device lengths O", o[:n], o_ref) <= 1.0
    assert report("split device lengths LSE", l[:, :n], l_ref) <= LSE_TOL
    assert np.all(o[n:] == 7.0) and np.all(l[:, n:] == 7.0)


@pytest.mark.parametrize("causal,with_prev", [(True, True), (True, False), (False, True)])
def test_split_two_row_lengths(mla, causal, with_prev):
    """[2, batch] lengths (MLA_SEQ_LENS_QK, Ascend seqLen's second form):
    each sequence's keys come from its own range of the key tensors.  The
    lengths cover more keys than queries, fewer (under TRIU the first
    Lq - Lk queries see no key), no keys, no queries (whose keys must still
    be skipped), one of each, and blocks past 128 rows."""
    ql = [130, 5, 0, 257, 64, 1, 200]
    kl = [300, 2, 7, 129, 0, 1, 450]
    c = W.split_case(seq_lens=ql, kv_lens=kl, H=4, Hkv=2, seed=91, with_prev=with_prev)
    out, o32, lse = _split_twin(mla, c, with_prev, causal=causal)
    o_ref, l_ref = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale, causal=causal,
                                    prev_out=c.prev_out if with_prev else None,
                                    prev_lse=c.prev_lse if with_prev else None)
    _twin("split two-row", out, o32, o_ref)
    assert report("split two-row LSE", host(lse), l_ref) <= LSE_TOL


def test_split_ring_step_over_a_past_chunk(mla):
    """The Ascend ring on split tensors: each sequence's current query chunk
    meets an earlier key chunk without a mask ([2, batch] lengths, a float32
    carry), then its own chunk under TRIU folded into that carry.  The result
    is the rows of the causal call over the whole sequences."""
    lens = [700, 300, 1200]
    past, cur = [(0, 400), (0, 100), (0, 512)], [(400, 700), (100, 300), (512, 1200)]
    c = W.split_case(seq_lens=lens, H=4, Hkv=2, seed=92, with_prev=False)
    cu = np.concatenate([[0], np.cumsum(lens)])
    qt = np.concatenate([np.arange(a, z) + cu[b] for b, (a, z) in enumerate(cur)])
    kt = np.concatenate([np.arange(a, z) + cu[b] for b, (a, z) in enumerate(past)])
    ql = np.array([z - a for a, z in cur], np.int32)
    kl = np.array([z - a for a, z in past], np.int32)
    g = lambda x, t: dev_bf16(np.ascontiguousarray(x[t]))
    q1, q2 = g(c.q1, qt), g(c.q2, qt)
    T, H = len(qt), c.q1.shape[1]
    carry = torch.empty((T, H, 128), dtype=torch.float32, device="cuda")
    o1, l1 = mla.split_fwd(q1, q2, g(c.k1, kt), g(c.k2, kt), g(c.v, kt), scale=c.scale,
                           seq_lens=dev(np.stack([ql, kl])), causal=False, out=carry)
    own = (q1, q2, g(c.k1, qt), g(c.k2, qt), g(c.v, qt))
    out, lse = mla.split_fwd(*own, scale=c.scale, seq_lens=dev(ql), causal=True, prev=(o1, l1))
    o32, l32 = mla.split_fwd(*own, scale=c.scale, seq_lens=dev(ql), causal=True, prev=(o1, l1),
                             out=torch.empty_like(carry))
    torch.cuda.synchronize()
    assert torch.equal(lse, l32)
    o_ref, l_ref = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale)
    _twin("split ring step", out, o32, o_ref[qt])
    assert report("split ring step LSE", host(lse), l_ref[:, qt]) <= LSE_TOL


def test_split_config_sampled(mla):
    """8 sequences (seed-0 lengths, T = 27610), 32 heads, prev fold: sampled
    tokens of each sequence for four heads against the oracle."""
    c = W.split_ring_step(0)
    out, o32, lse = _split_twin(mla, c)
    assert_rne_of("split cfg", out, o32)          # every element of the step
    cu = np.concatenate([[0], np.cumsum(c.seq_lens)])
    f = W.bf16_bits_to_f64
    worst_o = worst_o32 = worst_l = 0.0
    for s in range(len(c.seq_lens)):
        t0, L = int(cu[s]), int(c.seq_lens[s])
        rows = np.unique(np.array([0, 1, 2, 3, 127, 128, L // 2, L - 2, L - 1]).clip(0, L - 1))
        for h in (0, 9, 22, 31):
            q = np.concatenate([f(c.q1[t0 + rows, h]), f(c.q2[t0 + rows, h])], 1)
            k = np.concatenate([f(c.k1[t0:t0 + L, h]), f(c.k2[t0:t0 + L, h])], 1)
            o, l = oracle.attention(q, k, f(c.v[t0:t0 + L, h]), c.scale, True, rows, np.arange(L))
            o, l = oracle.merge(c.prev_out[t0 + rows, h], c.prev_lse[h, t0 + rows], o, l)
            worst_o = max(worst_o, report_o(f"split s{s} h{h} O", host(out[t0 + rows, h]), o))
            worst_o32 = max(worst_o32, report(f"split s{s} h{h} fp32 O", host(o32[t0 + rows, h]), o))
            worst_l = max(worst_l, report(f"split s{s} h{h} LSE", host(lse[h, t0 + rows]), l))
    assert worst_o <= 1.0 and worst_o32 <= O_TOL and worst_l <= LSE_TOL


# ---------------------------------------------------------------------------
# sparse top-k
# ---------------------------------------------------------------------------
def _sparse_gpu(mla, c, idx=None, out=None):
    idx = c.idx if idx is None else idx
    out, lse = mla.sparse_fwd(dev_bf16(c.q_lift), dev_bf16(c.q_pe), dev_bf16(c.c_kv),
                              dev_bf16(c.k_pe), dev(idx), scale=c.scale, out=out)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("H,K,seed", [(128, 96, 40), (20, 2048, 41), (128, 40, 42),
                                      (16, 2049, 46), (128, 1, 47), (8, 2900, 49),
                                      (24, 4096, 50)])   # the longest list the kernel takes
def test_sparse_small(mla, H, K, seed):
    c = W.sparse_case(S=24, S_kv=max(3000, K + 100), pos0=max(2900, K + 50), H=H, K=K, seed=seed)
    out, lse = _sparse_gpu(mla, c)
    o32, _ = _sparse_gpu(mla, c, out=_f32(out))
    o_ref, l_ref = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, c.idx, c.scale)
    _twin("sparse", out, o32, o_ref)
    assert report("sparse LSE", host(lse), l_ref) <= LSE_TOL


def test_sparse_mx4_output_order(mla):
    """MLA_OUT_MX4: the kernel's output equals the oracle's natural-order
    result put through the MX 4-pack permutation, and the natural-order call
    permuted the same way is bit-identical to it."""
    c = W.sparse_case(S=24, S_kv=3000, pos0=2900, H=128, K=700, seed=88)
    args = [dev_bf16(x) for x in (c.q_lift, c.q_pe, c.c_kv, c.k_pe)] + [dev(c.idx)]
    o_mx, l_mx = mla.sparse_fwd(*args, scale=c.scale, mx4=True)
    o_nat, l_nat = mla.sparse_fwd(*args, scale=c.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, c.idx, c.scale)
    assert report_o("mx4 O", host(o_mx), oracle.mx4_pack(o_ref, 512)) <= 1.0
    assert report("mx4 LSE", host(l_mx), l_ref) <= LSE_TOL
    perm = oracle.mx4_pack(np.arange(512, dtype=np.float64), 512).astype(np.int64)
    nat = o_nat.view(torch.int16).view(1, 24, 128, 512).cpu().numpy()
    want = np.empty_like(nat)
    want[..., np.arange(512)] = nat[..., perm]
    assert np.array_equal(o_mx.view(torch.int16).view(1, 24, 128, 512).cpu().numpy(), want)
    assert torch.equal(l_mx, l_nat)


def test_sparse_duplicates_and_invalid_indices(mla):
    c = W.sparse_case(S=8, S_kv=500, pos0=300, H=128, K=64, seed=43)
    idx = c.idx.copy()
    idx[0, 0, 10:20] = idx[0, 0, 3]          # repeats count with multiplicity
    idx[0, 1, 5] = -1                        # skipped
    idx[0, 2, 7] = 500                       # past the cache: skipped
    idx[0, 3, :] = -1                        # nothing valid: O = 0, LSE = -inf
    out, lse = _sparse_gpu(mla, c, idx)
    o_ref, l_ref = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, idx, c.scale)
    assert report_o("sparse dup O", host(out), o_ref) <= 1.0
    assert report("sparse dup LSE", host(lse), l_ref) <= LSE_TOL


def test_sparse_repeated_row_bit_exact(mla):
    """K copies of one row: every weight is 1, so out = c_kv[r] exactly and
    LSE = s_r + ln K."""
    c = W.sparse_case(S=6, S_kv=400, pos0=300, H=128, K=256, seed=44)
    r = 123
    idx = np.full_like(c.idx, r)
    out, lse = _sparse_gpu(mla, c, idx)
    got = out.view(torch.int16).cpu().numpy().reshape(6, 128, 512)
    want = np.broadcast_to(c.c_kv[0, r].view(np.int16), (6, 128, 512))
    assert np.array_equal(got, want)
    _, l_ref = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, idx, c.scale)
    assert report("repeated LSE", host(lse), l_ref) <= LSE_TOL


def test_debug_gather_bit_exact(mla):
    c = W.sparse_case(S=2, S_kv=1000, pos0=900, H=4, K=200, seed=45)
    ck, kp = dev_bf16(c.c_kv), dev_bf16(c.k_pe)
    idx = c.idx[0, 1].copy()
    idx[7] = -3
    idx[8] = 1000
    rows = mla.debug_gather(ck, kp, dev(idx))
    torch.cuda.synchronize()
    cat = torch.cat([ck[0], kp[0]], dim=1)
    safe = torch.from_numpy(np.where((idx >= 0) & (idx < 1000), idx, 0).astype(np.int64)).cuda()
    want = cat.index_select(0, safe)
    want[7] = 0
    want[8] = 0
    assert torch.equal(rows.view(torch.int16), want.view(torch.int16))


def test_sparse_config_sampled(mla):
    """S = 4096 queries at positions 12288.., 16384 cache rows, 128 heads,
    K = 2048: sampled queries (all heads) against the oracle."""
    c = W.sparse_topk(0)
    out, lse = _sparse_gpu(mla, c)
    rows = [0, 1, 1000, 2047, 4094, 4095]
    o_ref, l_ref = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, c.idx, c.scale, rows=rows)
    assert report_o("sparse cfg O", host(out[:, rows]), o_ref) <= 1.0
    assert report("sparse cfg LSE", host(lse[:, rows]), l_ref) <= LSE_TOL


# ---------------------------------------------------------------------------
# wide score range: the row maxima grow far past the reference max that the
# kernels fix at a row's first key tile, so every form takes its second,
# exact-max pass.  The 64 RoPE columns of queries and keys are scaled by 8
# (exact in bf16), which gives scores of about 37 nats standard deviation.
# The weights are then close to one-hot, so an output is close to one value
# row and reaches |O| > 4; the float32 twins hold the arithmetic to 1e-2.
# ---------------------------------------------------------------------------
def _times_pow2(bits, f, cols=slice(None)):
    """bf16 bits with the columns `cols` of the last axis times a power of two
    (exact: only the exponent changes)."""
    x = W.bf16_bits_to_f32(bits)
    x[..., cols] *= np.float32(f)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _max_growth_log2(q, k, scale, vis):
    """Largest growth, in log2 units, of a row's score max over the max of its
    first 32 visible keys.  q [R, d], k [n, d] (fp64), vis [R, n] bool."""
    s = (q @ k.T) * scale / math.log(2.0)
    s = np.where(vis, s, -np.inf)
    first = np.array([row[v][:32].max() if v.any() else -np.inf for row, v in zip(s, vis)])
    full = s.max(axis=1)
    ok = np.isfinite(first)
    return float((full[ok] - first[ok]).max())


def test_dense_wide_range_second_pass(mla):
    c = W.dense_case(B=1, H=6, N=200, seed=8)
    c.q = _times_pow2(c.q, 8.0, slice(512, None))
    c.kv = _times_pow2(c.kv, 8.0, slice(512, None))
    q64, k64 = W.bf16_bits_to_f64(c.q[0, 0]), W.bf16_bits_to_f64(c.kv[0, 0])
    vis = np.tril(np.ones((200, 200), dtype=bool))
    assert _max_growth_log2(q64, k64, c.scale, vis) > 40.0
    out, lse = _dense_gpu(mla, c)
    o32, l32 = _dense_gpu(mla, c, out=_f32(out))
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    _twin("wide", out, o32, o_ref)
    assert report("wide LSE", host(lse), l_ref) <= LSE_TOL
    assert torch.equal(lse, l32)


@pytest.mark.parametrize("K", [300, 2400])
def test_sparse_wide_range_second_pass(mla, K):
    c = W.sparse_case(S=8, S_kv=3000, pos0=2900, H=32, K=K, seed=50 + K)
    c.q_pe = _times_pow2(c.q_pe, 8.0)
    c.k_pe = _times_pow2(c.k_pe, 8.0)
    q64 = np.concatenate([W.bf16_bits_to_f64(c.q_lift[0, 0]), W.bf16_bits_to_f64(c.q_pe[0, 0])], axis=1)
    rows = np.concatenate([W.bf16_bits_to_f64(c.c_kv[0]), W.bf16_bits_to_f64(c.k_pe[0])], axis=1)
    k64 = rows[c.idx[0, 0]]
    assert _max_growth_log2(q64, k64, c.scale, np.ones((32, K), dtype=bool)) > 40.0
    out, lse = _sparse_gpu(mla, c)
    o32, l32 = _sparse_gpu(mla, c, out=torch.empty(out.shape, dtype=torch.float32, device="cuda"))
    o_ref, l_ref = oracle.sparse_mla(c.q_lift, c.q_pe, c.c_kv, c.k_pe, c.idx, c.scale)
    _twin("wide sparse", out, o32, o_ref)
    assert report("wide sparse LSE", host(lse), l_ref) <= LSE_TOL
    assert torch.equal(lse, l32)


def test_split_wide_range_second_pass(mla):
    c = W.split_case(seq_lens=[300, 77], H=4, Hkv=2, seed=9, with_prev=True)
    c.q2 = _times_pow2(c.q2, 8.0)
    c.k2 = _times_pow2(c.k2, 8.0)
    q64 = np.concatenate([W.bf16_bits_to_f64(c.q1[:300, 0]), W.bf16_bits_to_f64(c.q2[:300, 0])], axis=1)
    k64 = np.concatenate([W.bf16_bits_to_f64(c.k1[:300, 0]), W.bf16_bits_to_f64(c.k2[:300, 0])], axis=1)
    assert _max_growth_log2(q64, k64, c.scale, np.tril(np.ones((300, 300), dtype=bool))) > 40.0
    out, o32, lse = _split_twin(mla, c, True)
    o_ref, l_ref = oracle.split_mla(c.q1, c.q2, c.k1, c.k2, c.v, c.seq_lens, c.scale,
                                    prev_out=c.prev_out, prev_lse=c.prev_lse)
    _twin("wide split", out, o32, o_ref)
    assert report("wide split LSE", host(lse), l_ref) <= LSE_TOL


# ---------------------------------------------------------------------------
# scale <= 0: the kernels scale and mask the scores before the softmax
# (rather than folding the scale into the exponent), so that the row max is
# taken on the scaled values; scale 0 gives uniform weights over the visible
# keys (the prefix mean of V, LSE = ln #visible)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("scale", [0.0, -0.05])
def test_non_positive_scale_all_forms(mla, scale):
    c = W.dense_case(B=1, H=5, N=150, Nkv=170, seed=60, q_offset=20)
    out, lse = mla.fwd(dev_bf16(c.q), dev_bf16(c.kv), scale=scale, q_offset=20)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, scale, q_offset=20)
    assert report_o(f"scale {scale} dense O", host(out), o_ref) <= 1.0
    assert report(f"scale {scale} dense LSE", host(lse), l_ref) <= LSE_TOL
    cs = W.sparse_case(S=6, S_kv=900, pos0=700, H=16, K=300, seed=61)
    o, l = mla.sparse_fwd(*[dev_bf16(x) for x in (cs.q_lift, cs.q_pe, cs.c_kv, cs.k_pe)], dev(cs.idx),
                          scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_mla(cs.q_lift, cs.q_pe, cs.c_kv, cs.k_pe, cs.idx, scale)
    assert report_o(f"scale {scale} sparse O", host(o), o_ref) <= 1.0
    assert report(f"scale {scale} sparse LSE", host(l), l_ref) <= LSE_TOL
    cp = W.split_case(seq_lens=[90, 160], H=4, Hkv=2, seed=62, with_prev=True)
    out, o32, lse = _split_twin(mla, cp, True, scale=scale)
    o_ref, l_ref = oracle.split_mla(cp.q1, cp.q2, cp.k1, cp.k2, cp.v, cp.seq_lens, scale,
                                    prev_out=cp.prev_out, prev_lse=cp.prev_lse)
    _twin(f"scale {scale} split", out, o32, o_ref)
    assert report(f"scale {scale} split LSE", host(lse), l_ref) <= LSE_TOL


# ---------------------------------------------------------------------------
# item queue: with a workspace, workgroups take their row blocks from a
# device counter instead of their launch index; every block is computed the
# same way, so the results are bit-identical
# ---------------------------------------------------------------------------
def test_dense_queue_bit_identical_to_launch_order(mla):
    """B = 2, 64 heads, N = 2048: 2048 row blocks, enough for the queue."""
    c = W.dense_case(B=2, H=64, N=2048, seed=12)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    ws = torch.empty(int(mla.binding.LIB.mla_workspace_size()), dtype=torch.uint8, device="cuda")
    o1, l1 = mla.fwd(q, kv, scale=c.scale, workspace=None)
    o2, l2 = mla.fwd(q, kv, scale=c.scale, workspace=ws)
    o3, l3 = mla.fwd(q, kv, scale=c.scale, workspace=ws)   # the counter is reset per call
    torch.cuda.synchronize()
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(l, l1)
    # and against the oracle on a few rows of the last batch
    b, heads, rows = 1, [0, 63], [0, 1000, 2047]
    for hh in heads:
        o_ref, l_ref = oracle.dense_mla(c.q[b:b + 1, hh:hh + 1], c.kv[b:b + 1], 512, c.scale, rows=rows)
        assert report_o("queue O", host(o2[b:b + 1, hh:hh + 1, rows]), o_ref) <= 1.0
        assert report("queue LSE", host(l2[b:b + 1, hh:hh + 1, rows]), l_ref) <= LSE_TOL


def test_sparse_queue_bit_identical_to_launch_order(mla):
    c = W.sparse_case(S=1100, S_kv=3000, pos0=1800, H=16, K=64, seed=13)
    args = (dev_bf16(c.q_lift), dev_bf16(c.q_pe), dev_bf16(c.c_kv), dev_bf16(c.k_pe), dev(c.idx))
    o1, l1 = mla.sparse_fwd(*args, scale=c.scale, workspace=None)
    o2, l2 = mla.sparse_fwd(*args, scale=c.scale, workspace="auto")
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(l2, l1)


# ---------------------------------------------------------------------------
# token generation (decode) with the keys split across workgroups
# ---------------------------------------------------------------------------
def _decode_gpu(mla, c, **kw):
    out, lse = mla.decode_fwd(dev_bf16(c.q), dev_bf16(c.kv), scale=c.scale,
                              kv_lens=dev(c.kv_lens), **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("B,H,Nkv,lens,n_splits", [
    (5, 128, 3000, [0, 1, 33, 2049, 3000], 0),    # library's split: 12 ranges of 256
    (5, 128, 3000, [0, 1, 33, 2049, 3000], 2),    # 2 ranges of 1504
    (3, 128, 2000, [2000, 700, 31], 1),           # one range: the attention kernel writes out
    (4, 16, 1100, [1100, 1, 500, 1099], 0),       # fewer heads
    (2, 128, 9000, [9000, 4500], 0),              # more than 2048 rows: several ranges at least
])
def test_decode_small(mla, B, H, Nkv, lens, n_splits):
    c = W.decode_case(B=B, H=H, Nkv=Nkv, kv_lens=lens, seed=70 + B + Nkv)
    out, lse = _decode_gpu(mla, c, n_splits=n_splits)
    o_ref, l_ref = oracle.decode_mla(c.q, c.kv, c.kv_lens, 512, c.scale)
    assert report_o("decode O", host(out), o_ref) <= 1.0
    assert report("decode LSE", host(lse), l_ref) <= LSE_TOL


@pytest.mark.parametrize("n_splits", [0, 2])
def test_decode_lengths_clamped_and_rows_past_them_unread(mla, n_splits):
    """kv_lens outside [0, Nkv] are clamped (-5 reads nothing, 5000 reads all
    3000 rows), and cache rows past a sequence's valid length are never read:
    NaN there (bf16 0x7fc0) leaves the result bitwise that of the clean
    cache."""
    c = W.decode_case(B=4, H=16, Nkv=3000, kv_lens=[-5, 5000, 17, 2048], seed=76)
    dirty = c.kv.copy()
    for b, n in enumerate(np.clip(c.kv_lens, 0, 3000)):
        dirty[b, n:] = 0x7fc0
    q, lens = dev_bf16(c.q), dev(c.kv_lens)
    o1, l1 = mla.decode_fwd(q, dev_bf16(c.kv), scale=c.scale, kv_lens=lens, n_splits=n_splits)
    o2, l2 = mla.decode_fwd(q, dev_bf16(dirty), scale=c.scale, kv_lens=lens, n_splits=n_splits)
    torch.cuda.synchronize()
    assert not torch.isnan(o2).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, l_ref = oracle.decode_mla(c.q, c.kv, np.clip(c.kv_lens, 0, 3000), 512, c.scale)
    assert report_o("decode clamped O", host(o1), o_ref) <= 1.0
    assert report("decode clamped LSE", host(l1), l_ref) <= LSE_TOL


def test_decode_split_rope_tensors_bit_identical(mla):
    """q/kv as one 576-column tensor or as 512 + 64 column tensors: the same
    bits."""
    c = W.decode_case(B=3, H=128, Nkv=1500, kv_lens=[1500, 900, 64], seed=75)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    lens = dev(c.kv_lens)
    o1, l1 = mla.decode_fwd(q, kv, scale=c.scale, kv_lens=lens)
    o2, l2 = mla.decode_fwd(q[..., :512].contiguous(), kv[..., :512].contiguous(), scale=c.scale, kv_lens=lens,
                            q_rope=q[..., 512:].contiguous(), k_rope=kv[..., 512:].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_decode_config_sampled(mla):
    """B = 64 sequences, 128 heads, 8192 cache rows each (the benchmarked
    launch: 4 ranges of 2048 per sequence): sampled sequences, all heads."""
    c = W.dsv3_decode(0)
    out, lse = _decode_gpu(mla, c)
    seqs = [0, 31, 63]
    o_ref, l_ref = oracle.decode_mla(c.q[seqs], c.kv[seqs], c.kv_lens[seqs], 512, c.scale)
    assert report_o("decode cfg O", host(out[seqs]), o_ref) <= 1.0
    assert report("decode cfg LSE", host(lse[seqs]), l_ref) <= LSE_TOL


# ---------------------------------------------------------------------------
# several calls in one launch (a ring step for all query chunks)
# ---------------------------------------------------------------------------
def test_group_bit_identical_to_separate_calls(mla):
    """Calls of different shapes, offsets, masks and fold options in one
    mla_fwd_group launch give the same bits as one mla_fwd each."""
    c = W.dense_case(B=2, H=8, N=600, Nkv=900, seed=80)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    g = torch.Generator().manual_seed(81)
    p_out = torch.randn((2, 8, 100, 512), generator=g).cuda()            # fp32 running output
    p_lse = (torch.rand((2, 8, 100), generator=g) * 8).cuda()
    def calls():
        return [dict(q=q[:, :, :256], kv=kv[:, :, :300], scale=c.scale, causal=True, q_offset=44),
                dict(q=q[:, :5, 256:], kv=kv[:, :, 300:], scale=c.scale, causal=False),
                dict(q=q[:, :, 100:200], kv=kv, scale=c.scale, causal=True, q_offset=800,
                     prev=(p_out, p_lse), out=torch.empty_like(p_out)),
                dict(q=q[:1, :, :33], kv=kv[:1, :, :40], scale=c.scale, causal=True, q_offset=7)]
    grouped = mla.fwd_group(calls())
    separate = [mla.fwd(workspace=None, **k) for k in calls()]
    torch.cuda.synchronize()
    for (og, lg), (os_, ls) in zip(grouped, separate):
        assert og.dtype == os_.dtype
        assert torch.equal(og.view(torch.int16) if og.dtype == torch.bfloat16 else og.view(torch.int32),
                           os_.view(torch.int16) if os_.dtype == torch.bfloat16 else os_.view(torch.int32))
        assert torch.equal(lg, ls)


def test_group_equal_calls_interleaved_bit_identical(mla):
    """Calls with equal workgroup counts take workgroups in turn; still the
    same bits as separate calls (here: the three query chunks of a ring step
    with different KV chunks, prev folds and both output types)."""
    c = W.dense_case(B=1, H=8, N=384, seed=82)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    g = torch.Generator().manual_seed(83)
    prev = [(torch.randn((1, 8, 128, 512), generator=g).cuda(), (torch.rand((1, 8, 128), generator=g) * 6).cuda())
            for _ in range(3)]
    def calls():
        return [dict(q=q[:, :, 128 * r:128 * (r + 1)], kv=kv[:, :, 128 * k:128 * (k + 1)], scale=c.scale,
                     causal=True, q_offset=128 * r, kv_offset=128 * k, prev=prev[r],
                     out=torch.empty((1, 8, 128, 512), dtype=torch.float32 if r else torch.bfloat16,
                                     device="cuda"))
                for r, k in ((0, 0), (1, 0), (2, 1))]
    grouped = mla.fwd_group(calls())
    separate = [mla.fwd(workspace=None, **k) for k in calls()]
    torch.cuda.synchronize()
    for (og, lg), (os_, ls) in zip(grouped, separate):
        view = torch.int16 if og.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(og.view(view), os_.view(view))
        assert torch.equal(lg, ls)


def test_decode_indexed_cache_slots(mla):
    """Sequences read cache slots through kv_slots (an indexed cache): two
    sequences share slot 3, one slot is out of range (no valid rows)."""
    rng = np.random.default_rng(84)
    q = W.normal_bf16(rng, (4, 128, 576))
    kv = W.normal_bf16(rng, (5, 2500, 576))
    slots = np.array([3, 0, 3, 7], dtype=np.int32)
    lens = np.array([2500, 640, 1200, 2500], dtype=np.int32)
    out, lse = mla.decode_fwd(dev_bf16(q), dev_bf16(kv), scale=W.SCALE_192, kv_lens=dev(lens),
                              kv_slots=dev(slots))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_mla(q, kv, lens, 512, W.SCALE_192, kv_slots=slots)
    assert report_o("slots O", host(out), o_ref) <= 1.0
    assert report("slots LSE", host(lse), l_ref) <= LSE_TOL


def test_split_workspace_bit_identical(mla):
    """Split varlen step (1888 row blocks) with and without a workspace."""
    c = W.split_case(seq_lens=[3000, 2500, 1800], H=32, Hkv=32, seed=85, with_prev=True)
    args = [dev_bf16(x) for x in (c.q1, c.q2, c.k1, c.k2, c.v)]
    sl = dev(c.seq_lens)
    prev = (dev_bf16(c.prev_out), dev(c.prev_lse))
    o1, l1 = mla.split_fwd(*args, scale=c.scale, seq_lens=sl, prev=prev, workspace=None)
    o2, l2 = mla.split_fwd(*args, scale=c.scale, seq_lens=sl, prev=prev, workspace="auto")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,N,lens,seed", [
    (3, 8, 300, [300, 77, 0], 86),         # full, ragged tail inside a row block, empty
    (2, 128, 1100, [1037, 5000], 87),      # 128 heads; a length past N clamps to N
])
def test_dense_valid_lens_padded_batch(mla, B, H, N, lens, seed):
    """Padded batch with per-batch valid lengths (MLA_VALID_LENS): batch b
    equals the oracle on its first lens[b] rows; rows past it are untouched.
    Rows that see only a few keys reach |O| > 2, so the float32 twin runs
    too."""
    c = W.dense_case(B=B, H=H, N=N, seed=seed)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    vl = dev(np.array(lens, dtype=np.int32))
    out = torch.full((B, H, N, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), 7.0, dtype=torch.float32, device="cuda")
    mla.fwd(q, kv, scale=c.scale, out=out, lse=lse, valid_lens=vl)
    o32 = torch.full((B, H, N, 512), 7.0, dtype=torch.float32, device="cuda")
    mla.fwd(q, kv, scale=c.scale, out=o32, lse=torch.empty_like(lse), valid_lens=vl)
    torch.cuda.synchronize()
    assert_rne_of("valid lens", out, o32)
    o, o_f, l = host(out), host(o32), host(lse)
    for b, n in enumerate(lens):
        n = min(n, N)
        if n:
            o_ref, l_ref = oracle.dense_mla(c.q[b:b + 1, :, :n], c.kv[b:b + 1, :, :n], 512, c.scale)
            assert report(f"b{b} fp32 O", o_f[b:b + 1, :, :n], o_ref) <= O_TOL
            assert report_o(f"b{b} O", o[b:b + 1, :, :n], o_ref) <= 1.0
            assert report(f"b{b} LSE", l[b:b + 1, :, :n], l_ref) <= LSE_TOL
        assert np.all(o[b, :, n:] == 7.0) and np.all(l[b, :, n:] == 7.0) and np.all(o_f[b, :, n:] == 7.0)


# ---------------------------------------------------------------------------
# V-up projection
# ---------------------------------------------------------------------------
def _vup_ok(name, got, ref):
    """Element-wise bound: the bf16 rounding of the result (at most 2^-8 of
    its magnitude) plus the fp32 accumulation over 512 products (at most
    512 * 2^-24 * sum |o w|, below 1e-3 for these inputs, where sum |o w| is
    about 512 * 0.8 * 0.035)."""
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    print(f"{name}: max err {err.max():.3e}, worst vs bound {err[worst]:.3e} <= {bound[worst]:.3e} at {worst}")
    return bool(np.all(err <= bound))


@pytest.mark.parametrize("B,H,T,seed", [(2, 5, 77, 90), (3, 128, 1, 91), (1, 16, 300, 92)])
def test_vup_small(mla, B, H, T, seed):
    """Every element; ragged row blocks, rows of several batches in one block
    (T = 1, the decode shape)."""
    c = W.vup_case(B=B, H=H, T=T, seed=seed)
    out = mla.vup(dev_bf16(c.o), dev_bf16(c.w_uv))
    torch.cuda.synchronize()
    ref = oracle.vup(c.o, c.w_uv)
    assert _vup_ok("vup", host(out).transpose(0, 2, 1, 3), ref)


def test_vup_sparse_layout_mx4(mla):
    """Input in the sparse output's [B, S, H*L] layout with MX 4-pack
    columns (a strided view), result equal to the natural projection."""
    c = W.vup_case(B=1, H=128, T=40, seed=93)
    packed = oracle.mx4_pack(W.bf16_bits_to_f32(c.o), 512)            # exact: a permutation
    flat = np.ascontiguousarray(packed.transpose(0, 2, 1, 3)).reshape(1, 40, 128 * 512)
    o = torch.from_numpy(flat).cuda().to(torch.bfloat16)
    out = mla.vup(o.view(1, 40, 128, 512).transpose(1, 2), dev_bf16(c.w_uv), mx4=True)
    torch.cuda.synchronize()
    assert _vup_ok("vup mx4", host(out).transpose(0, 2, 1, 3), oracle.vup(c.o, c.w_uv))


def test_vup_config_sampled(mla):
    """The V-up workload the benchmark times (H = 128, T = 8192): sampled
    rows against the oracle, row by row."""
    c = W.dsv3_vup(0)
    out = mla.vup(dev_bf16(c.o), dev_bf16(c.w_uv))
    torch.cuda.synchronize()
    rng = np.random.default_rng(94)
    hs = rng.integers(0, 128, 48)
    ts = np.concatenate([rng.integers(0, 8192, 46), [0, 8191]])
    got = out[0, torch.from_numpy(ts), torch.from_numpy(hs)].float().cpu().numpy().astype(np.float64)
    ref = np.stack([oracle.vup(c.o[:, h:h + 1, t:t + 1], c.w_uv[h:h + 1])[0, 0, 0] for h, t in zip(hs, ts)])
    assert _vup_ok("vup config", got, ref)


# ---------------------------------------------------------------------------
# degenerate and extreme sizes
# ---------------------------------------------------------------------------
def test_empty_sizes(mla):
    """Empty inputs: no query rows, no batches, no key rows (every row sees
    nothing: O = 0 and LSE = -inf, and a fold leaves the previous result as it
    is), and empty merge, sparse, V-up and decode calls.  An empty GPU tensor
    has a NULL data pointer, which the library accepts for a view that holds
    no rows."""
    rng = np.random.default_rng(95)
    z = lambda *shape: torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    sc = W.SCALE_192
    q = dev_bf16(W.normal_bf16(rng, (1, 4, 40, 576)))
    kv = dev_bf16(W.normal_bf16(rng, (1, 1, 64, 576)))
    out, lse = mla.fwd(z(1, 4, 0, 576), kv, scale=sc)                  # no query rows
    assert out.shape == (1, 4, 0, 512) and lse.shape == (1, 4, 0)
    out, lse = mla.fwd(z(0, 4, 40, 576), z(0, 1, 64, 576), scale=sc)   # no batches
    assert out.shape == (0, 4, 40, 512)
    for causal in (True, False):                                       # no key rows
        out, lse = mla.fwd(q, z(1, 1, 0, 576), scale=sc, causal=causal)
        torch.cuda.synchronize()
        assert (host(out) == 0).all() and np.isneginf(host(lse)).all()
    p_out = dev_bf16(W.normal_bf16(rng, (1, 4, 40, 512)))
    p_lse = dev(rng.uniform(0, 12, (1, 4, 40)).astype(np.float32))
    out, lse = mla.fwd(q, z(1, 1, 0, 576), scale=sc, prev=(p_out, p_lse))
    torch.cuda.synchronize()
    assert torch.equal(out, p_out) and torch.equal(lse, p_lse)         # the fold identity
    e = z(1, 4, 0, 512)
    el = torch.empty((1, 4, 0), dtype=torch.float32, device="cuda")
    mo, ml = mla.merge(e, el, e, el)                                   # merge of no rows
    assert mo.shape == (1, 4, 0, 512)
    idx = torch.empty((1, 0, 128), dtype=torch.int32, device="cuda")
    so, sl = mla.sparse_fwd(z(1, 0, 16, 512), z(1, 0, 16, 64), dev_bf16(W.normal_bf16(rng, (1, 300, 512))),
                            dev_bf16(W.normal_bf16(rng, (1, 300, 64))), idx, scale=sc)
    assert so.shape == (1, 0, 16 * 512)
    w = dev_bf16(W.normal_bf16(rng, (4, 128, 512)))
    vo = mla.vup(z(1, 4, 0, 512), w)                                   # V-up of no rows
    assert vo.numel() == 0
    do, dl = mla.decode_fwd(z(0, 16, 576), z(0, 100, 576), scale=sc)   # no sequences
    assert do.shape == (0, 16, 512)
    do, dl = mla.decode_fwd(dev_bf16(W.normal_bf16(rng, (2, 16, 576))), z(2, 0, 576), scale=sc)  # no cache rows
    torch.cuda.synchronize()
    assert (host(do) == 0).all() and np.isneginf(host(dl)).all()


def test_decode_longest_cache(mla):
    """The longest cache decode takes: 131,072 rows in 64 ranges of 2048, one
    sequence at full length and one ragged, against the oracle."""
    c = W.decode_case(B=2, H=128, Nkv=131072, kv_lens=[131072, 100001], seed=96)
    out, lse = mla.decode_fwd(dev_bf16(c.q), dev_bf16(c.kv), scale=c.scale, kv_lens=dev(c.kv_lens))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_mla(c.q, c.kv, c.kv_lens, 512, c.scale)
    assert report_o("decode 131072 O", host(out), o_ref) <= 1.0
    assert report("decode 131072 LSE", host(lse), l_ref) <= LSE_TOL


def test_ring_hip_graph_replays_match_eager(mla):
    """The ring driver captured in a HIP graph (it allocates nothing and
    records no memset: a kernel clears the item counter):
    several replays, with eager work and synchronisations between them, each
    bit-identical to the eager result."""
    c = W.dense_case(B=1, H=8, N=1024, seed=97)
    q, kv = dev_bf16(c.q), dev_bf16(c.kv)
    out = torch.empty((1, 8, 1024, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 8, 1024), dtype=torch.float32, device="cuda")
    carry = torch.empty(mla.ring_workspace_size(1, 8, 1024, 4), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # the eager result, off the capture stream
        mla.ring_fwd(q, kv, 4, scale=c.scale, out=out, lse=lse, carry=carry)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    o_eager, l_eager = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mla.ring_fwd(q, kv, 4, scale=c.scale, out=out, lse=lse, carry=carry)
    for rep in range(3):
        out.fill_(0)
        lse.fill_(0)
        mla.fwd(q, kv, scale=c.scale)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, o_eager), f"replay {rep}: O differs from eager"
        assert torch.equal(lse, l_eager), f"replay {rep}: LSE differs from eager"
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    assert report_o("graph ring O", host(out), o_ref) <= 1.0
    assert report("graph ring LSE", host(lse), l_ref) <= LSE_TOL


def test_ring_two_batches_strided_q(mla):
    """The native ring driver with B = 2 (batch strides through every chunk
    view) and q a strided view (every other head of a larger tensor), both
    schedules, against the unchunked oracle."""
    c = W.dense_case(B=2, H=6, N=384, seed=98)
    q_all = dev_bf16(c.q)
    big = torch.zeros((2, 12, 384, 576), dtype=torch.bfloat16, device="cuda")
    big[:, ::2] = q_all
    q_view = big[:, ::2]                       # stride_h twice the contiguous one
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale)
    for order in ("ring", "balanced"):
        out, lse = mla.ring_fwd(q_view, dev_bf16(c.kv), 3, scale=c.scale, order=order)
        torch.cuda.synchronize()
        assert report_o(f"ring B=2 {order} O", host(out), o_ref) <= 1.0
        assert report(f"ring B=2 {order} LSE", host(lse), l_ref) <= LSE_TOL


# ---------------------------------------------------------------------------
# randomized shapes (fixed seeds): every form against the oracle
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_all_forms(mla, seed):
    """Random sizes, offsets, masks, head groupings, sequence lengths (zero
    included), prev folds and decode valid lengths, drawn from a fixed seed:
    the dense, sparse, split (one- and two-row lengths, and batched views
    with offsets), decode and ring forms against the oracle."""
    r = np.random.default_rng(1000 + seed)
    # dense: batches, heads, query and key counts, offsets, mask
    B, H = int(r.integers(1, 3)), int(r.integers(1, 10))
    N, Nkv = int(r.integers(1, 300)), int(r.integers(1, 400))
    causal = bool(r.integers(0, 2))
    qo, ko = int(r.integers(0, 300)), int(r.integers(0, 200))
    c = W.dense_case(B=B, H=H, N=N, Nkv=Nkv, seed=seed, causal=causal, q_offset=qo, kv_offset=ko)
    o, l = mla.fwd(dev_bf16(c.q), dev_bf16(c.kv), scale=c.scale, causal=causal, q_offset=qo, kv_offset=ko)
    o32, _ = mla.fwd(dev_bf16(c.q), dev_bf16(c.kv), scale=c.scale, causal=causal, q_offset=qo, kv_offset=ko,
                     out=_f32(o))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.dense_mla(c.q, c.kv, 512, c.scale, causal=causal, q_offset=qo, kv_offset=ko)
    _twin("random dense", o, o32, o_ref)
    assert report("random dense LSE", host(l), l_ref) <= LSE_TOL
    # sparse: queries, list length, heads
    S, K, Hs = int(r.integers(1, 20)), int(r.integers(1, 700)), int(r.integers(1, 129))
    cs = W.sparse_case(S=S, S_kv=K + 200, pos0=K + 50, H=Hs, K=K, seed=seed)
    o, l = _sparse_gpu(mla, cs)
    o32, _ = _sparse_gpu(mla, cs, out=_f32(o))
    o_ref, l_ref = oracle.sparse_mla(cs.q_lift, cs.q_pe, cs.c_kv, cs.k_pe, cs.idx, cs.scale)
    _twin("random sparse", o, o32, o_ref)
    assert report("random sparse LSE", host(l), l_ref) <= LSE_TOL
    # split: sequence lengths (zero allowed), head grouping, prev fold
    lens = [int(x) for x in r.integers(0, 300, int(r.integers(1, 5)))]
    if sum(lens) == 0:
        lens[0] = 1
    Hsp = int(r.choice([2, 4, 8]))
    Hkv = int(r.choice([h for h in (1, 2, Hsp) if Hsp % h == 0]))
    cp = W.split_case(seq_lens=lens, H=Hsp, Hkv=Hkv, seed=seed, with_prev=bool(r.integers(0, 2)))
    o, o32, l = _split_twin(mla, cp)
    o_ref, l_ref = oracle.split_mla(cp.q1, cp.q2, cp.k1, cp.k2, cp.v, cp.seq_lens, cp.scale, causal=True,
                                    prev_out=cp.prev_out, prev_lse=cp.prev_lse)
    _twin("random split", o, o32, o_ref)
    assert report("random split LSE", host(l), l_ref) <= LSE_TOL
    # decode: sequences, heads, cache rows, valid lengths (zero allowed)
    Bd, Hd, Nd = int(r.integers(1, 6)), int(r.integers(1, 129)), int(r.integers(1, 5000))
    kl = [int(x) for x in r.integers(0, Nd + 1, Bd)]
    cd = W.decode_case(B=Bd, H=Hd, Nkv=Nd, kv_lens=kl, seed=seed)
    o, l = mla.decode_fwd(dev_bf16(cd.q), dev_bf16(cd.kv), scale=cd.scale, kv_lens=dev(cd.kv_lens))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_mla(cd.q, cd.kv, cd.kv_lens, 512, cd.scale)
    assert report_o("random decode O", host(o), o_ref) <= 1.0
    assert report("random decode LSE", host(l), l_ref) <= LSE_TOL
    # split with separate key lengths ([2, batch]; zeros allowed), with or without the mask
    nq = len(lens)
    ql2 = [int(x) for x in r.integers(0, 200, nq)]
    kl2 = [int(x) for x in r.integers(0, 260, nq)]
    ql2[0], kl2[0] = max(ql2[0], 1), max(kl2[0], 1)
    causal2 = bool(r.integers(0, 2))
    c2 = W.split_case(seq_lens=ql2, kv_lens=kl2, H=Hsp, Hkv=Hkv, seed=seed + 50, with_prev=bool(r.integers(0, 2)))
    o, o32, l = _split_twin(mla, c2, causal=causal2)
    o_ref, l_ref = oracle.split_mla(c2.q1, c2.q2, c2.k1, c2.k2, c2.v, c2.seq_lens, c2.scale, causal=causal2,
                                    prev_out=c2.prev_out, prev_lse=c2.prev_lse)
    _twin("random split two-row", o, o32, o_ref)
    assert report("random split two-row LSE", host(l), l_ref) <= LSE_TOL
    # the split form over [B, H, N, D] views: batches, head grouping, offsets, mask
    Bb, Nb, Nkb = int(r.integers(1, 3)), int(r.integers(1, 200)), int(r.integers(1, 260))
    qob, kob, cb = int(r.integers(0, 100)), int(r.integers(0, 100)), bool(r.integers(0, 2))
    qs = [W.normal_bf16(r, (Bb, Hsp, Nb, d)) for d in (128, 64)]
    ks = [W.normal_bf16(r, (Bb, Hkv, Nkb, d)) for d in (128, 64, 128)]
    kw = dict(scale=W.SCALE_192, causal=cb, q_offset=qob, kv_offset=kob, q_rope=dev_bf16(qs[1]),
              k_rope=dev_bf16(ks[1]), v=dev_bf16(ks[2]))
    o, l = mla.fwd(dev_bf16(qs[0]), dev_bf16(ks[0]), **kw)
    o32, _ = mla.fwd(dev_bf16(qs[0]), dev_bf16(ks[0]), out=_f32(o), **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.dense_mla(np.concatenate(qs, -1), np.concatenate(ks[:2], -1), 128, W.SCALE_192,
                                    causal=cb, q_offset=qob, kv_offset=kob, v=ks[2])
    _twin("random split batched", o, o32, o_ref)
    assert report("random split batched LSE", host(l), l_ref) <= LSE_TOL
    # the one-device ring: length, chunk count, heads, schedule
    Nr, P, Hr = int(r.integers(1, 600)), int(r.integers(1, 7)), int(r.integers(1, 9))
    order = str(r.choice(["ring", "balanced"]))
    cr = W.dense_case(B=1, H=Hr, N=Nr, seed=seed + 100)
    o, l = mla.ring_fwd(dev_bf16(cr.q), dev_bf16(cr.kv), P, scale=cr.scale, order=order)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.dense_mla(cr.q, cr.kv, 512, cr.scale)
    assert report_o(f"random ring P={P} {order} O", host(o), o_ref) <= 1.0
    assert report("random ring LSE", host(l), l_ref) <= LSE_TOL
