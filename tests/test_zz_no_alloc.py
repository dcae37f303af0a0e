"""mla_decode_fwd_noalloc: decode through the library's static device scratch
(no workspace, no allocation) gives the same bits as mla_decode_fwd with a
workspace, call after call on the same scratch, and matches the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import LSE_TOL, dev, dev_bf16, host, report, report_o

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mla():
    import ring_chunk_attention_amd as m
    return m


def _both(mla, c, **kw):
    """(out, lse) of the no-alloc call and of the workspace call on the same
    inputs; the no-alloc call's outputs are given, so nothing is allocated
    for it."""
    q, kv, lens = dev_bf16(c.q), dev_bf16(c.kv), dev(c.kv_lens)
    B, H = c.q.shape[:2]
    out = torch.full((B, H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), 3.0, dtype=torch.float32, device="cuda")
    mla.decode_fwd(q, kv, scale=c.scale, kv_lens=lens, out=out, lse=lse, noalloc=True, **kw)
    o_ws, l_ws = mla.decode_fwd(q, kv, scale=c.scale, kv_lens=lens, **kw)
    torch.cuda.synchronize()
    return out, lse, o_ws, l_ws


def test_noalloc_two_calls_match_workspace_entry_point(mla):
    """Call 1: the 64 x 8192-row batch in 4 key ranges (64 MiB of partials in
    the scratch).  Call 2, right after on the same scratch: a smaller ragged
    batch with a zero length and another split.  Each bit-identical to
    mla_decode_fwd and within the bounds against the oracle."""
    big = W.dsv3_decode(0)
    print("noalloc call 1: B=64 H=128 Nkv=8192", flush=True)
    o1, l1, w1, wl1 = _both(mla, big)
    assert torch.equal(o1.view(torch.int16), w1.view(torch.int16)) and torch.equal(l1, wl1)
    seqs = [0, 63]
    o_ref, l_ref = oracle.decode_mla(big.q[seqs], big.kv[seqs], big.kv_lens[seqs], 512, big.scale)
    assert report_o("noalloc call 1 O", host(o1[seqs]), o_ref) <= 1.0
    assert report("noalloc call 1 LSE", host(l1[seqs]), l_ref) <= LSE_TOL

    small = W.decode_case(B=5, H=16, Nkv=1300, kv_lens=[1300, 0, 1, 700, 1299], seed=301)
    print("noalloc call 2: B=5 H=16 Nkv=1300", flush=True)
    o2, l2, w2, wl2 = _both(mla, small)
    assert torch.equal(o2.view(torch.int16), w2.view(torch.int16)) and torch.equal(l2, wl2)
    o_ref, l_ref = oracle.decode_mla(small.q, small.kv, small.kv_lens, 512, small.scale)
    assert report_o("noalloc call 2 O", host(o2), o_ref) <= 1.0
    assert report("noalloc call 2 LSE", host(l2), l_ref) <= LSE_TOL


def test_noalloc_one_range_and_explicit_split(mla):
    """One key range (the attention kernel writes out itself) and a caller's
    split of 3, one after the other on the shared scratch."""
    c = W.decode_case(B=4, H=128, Nkv=2000, kv_lens=[2000, 33, 0, 1999], seed=302)
    for n in (1, 3):
        print(f"noalloc n_splits={n}", flush=True)
        o, l, w, wl = _both(mla, c, n_splits=n)
        assert torch.equal(o.view(torch.int16), w.view(torch.int16)) and torch.equal(l, wl)
    o_ref, l_ref = oracle.decode_mla(c.q, c.kv, c.kv_lens, 512, c.scale)
    assert report_o("noalloc split 3 O", host(o), o_ref) <= 1.0
    assert report("noalloc split 3 LSE", host(l), l_ref) <= LSE_TOL
