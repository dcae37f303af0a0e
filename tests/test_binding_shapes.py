"""The binding refuses tensors whose shape, dtype or device does not match
the sizes it passes to the C ABI (the library sees only pointers and sizes,
so such a call would read or write out of bounds).  Host only: the tensors
live on torch's "meta" device, which the binding is allowed to accept for
the duration of these tests; every case must fail with ValueError before
any library call."""
import pytest

torch = pytest.importorskip("torch")

import ring_chunk_attention_amd.binding as bd  # noqa: E402


@pytest.fixture(autouse=True)
def meta_ok(monkeypatch):
    real = bd._need

    def need(t, name, dtype):
        if isinstance(t, torch.Tensor) and t.device.type == "meta":
            if t.dtype != dtype:
                raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
            return
        real(t, name, dtype)

    def no_call(*a, **k):
        raise AssertionError("the library was called: the shape check let the call through")

    monkeypatch.setattr(bd, "_need", need)
    monkeypatch.setattr(bd, "_check", no_call)
    monkeypatch.setattr(bd, "_stream", lambda device: None)
    yield


def m(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="meta")


def f32(*shape):
    return m(*shape, dtype=torch.float32)


def i32(*shape):
    return m(*shape, dtype=torch.int32)


def rejected(fn, *a, match="expected", **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


# --------------------------------------------------------------------- fwd
Q, KV = (2, 4, 64, 576), (2, 1, 64, 576)


@pytest.mark.parametrize("kw", [
    dict(kv=m(1, 1, 64, 576)),                                   # kv batch != B
    dict(kv=m(2, 1, 64, 512)),                                   # kv width != q width
    dict(out=m(2, 4, 64, 256)),                                  # out columns
    dict(out=m(2, 4, 63, 512)),                                  # out rows
    dict(lse=f32(2, 4, 32)),                                     # lse rows
    dict(prev=(m(2, 4, 64, 512), f32(2, 3, 64))),                # prev_lse heads
    dict(prev=(m(1, 4, 64, 512), f32(2, 4, 64))),                # prev_out batch
    dict(q_rope=m(2, 4, 64, 64), k_rope=m(2, 1, 60, 64)),        # k_rope rows
    dict(q_rope=m(2, 4, 64, 64)),                                # k_rope missing
])
def test_fwd_mismatched_tensors(kw):
    base = dict(q=m(*Q), kv=m(*KV))
    base.update(kw)
    q, kv = base.pop("q"), base.pop("kv")
    rejected(bd.fwd, q, kv, scale=0.07, workspace=None, match="expected|both", **base)


def test_fwd_mismatched_valid_lens_and_explicit_v():
    rejected(bd.fwd, m(*Q), m(*KV), scale=0.07, workspace=None, valid_lens=i32(3))
    rejected(bd.fwd, m(2, 4, 64, 128), m(2, 2, 64, 128), scale=0.07, workspace=None, v=m(2, 2, 60, 128))


def test_fwd_group_mismatched_tensors():
    rejected(bd.fwd_group, [dict(q=m(*Q), kv=m(*KV), scale=0.07, out=m(2, 4, 64, 500))])


# ------------------------------------------------------------------- split
T, H, HKV = 50, 4, 2


def split_args(**over):
    a = dict(q1=m(T, H, 128), q2=m(T, H, 64), k1=m(T, HKV, 128), k2=m(T, HKV, 64), v=m(T, HKV, 128))
    a.update(over)
    return a


@pytest.mark.parametrize("over,kw", [
    (dict(q2=m(T, H, 32)), {}),
    (dict(k1=m(T - 1, HKV, 128)), {}),
    (dict(k2=m(T, HKV + 1, 64)), {}),
    (dict(v=m(T + 1, HKV, 128)), {}),
    ({}, dict(out=m(T, H, 64))),
    ({}, dict(lse=f32(T, H))),
    ({}, dict(prev=(m(T, H, 128), f32(H, T - 1)))),
    ({}, dict(prev=(f32(T, H + 1, 128), f32(H, T)))),
])
def test_split_mismatched_tensors(over, kw):
    a = split_args(**over)
    rejected(bd.split_fwd, a["q1"], a["q2"], a["k1"], a["k2"], a["v"], scale=0.07, workspace=None, **kw)


def test_split_two_row_lengths_take_other_key_counts():
    """With [2, batch] seq_lens the key tensors may hold another token count
    (the call reaches the library); the key tensors must still agree with one
    another, and seq_lens must have two rows."""
    a = split_args(k1=m(T + 7, HKV, 128), k2=m(T + 7, HKV, 64), v=m(T + 7, HKV, 128))
    with pytest.raises(AssertionError, match="library was called"):
        bd.split_fwd(a["q1"], a["q2"], a["k1"], a["k2"], a["v"], scale=0.07, workspace=None,
                     seq_lens=i32(2, 3))
    rejected(bd.split_fwd, a["q1"], a["q2"], a["k1"], a["k2"], a["v"], scale=0.07, workspace=None,
             seq_lens=i32(3))
    rejected(bd.split_fwd, a["q1"], a["q2"], a["k1"], a["k2"], a["v"], scale=0.07, workspace=None,
             seq_lens=i32(3, 3))
    b = split_args(k1=m(T + 7, HKV, 128), k2=m(T + 7, HKV, 64), v=m(T + 6, HKV, 128))
    rejected(bd.split_fwd, b["q1"], b["q2"], b["k1"], b["k2"], b["v"], scale=0.07, workspace=None,
             seq_lens=i32(2, 3))


def test_split_accepts_fp32_out_and_prev_up_to_the_library():
    """fp32 out and prev_out pass the binding's checks (the call then reaches
    the library, which the fixture turns into an AssertionError)."""
    a = split_args()
    with pytest.raises(AssertionError, match="library was called"):
        bd.split_fwd(a["q1"], a["q2"], a["k1"], a["k2"], a["v"], scale=0.07, workspace=None,
                     out=f32(T, H, 128), prev=(f32(T, H, 128), f32(H, T)))


# ------------------------------------------------------------------- merge
@pytest.mark.parametrize("which,bad", [
    ("out_b", m(1, 2, 9, 512)), ("lse_a", f32(1, 2, 8)), ("lse_b", f32(1, 3, 10)),
    ("out", m(1, 2, 10, 256)), ("lse", f32(2, 2, 10)),
])
def test_merge_mismatched_tensors(which, bad):
    a = dict(out_a=m(1, 2, 10, 512), lse_a=f32(1, 2, 10), out_b=m(1, 2, 10, 512), lse_b=f32(1, 2, 10))
    kw = {}
    if which in a:
        a[which] = bad
    else:
        kw[which] = bad
    rejected(bd.merge, a["out_a"], a["lse_a"], a["out_b"], a["lse_b"], **kw)


# ------------------------------------------------------------------ sparse
def test_sparse_mismatched_tensors():
    ql, qp, ck, kp, ix = m(1, 8, 16, 512), m(1, 8, 16, 64), m(1, 300, 512), m(1, 300, 64), i32(1, 8, 32)
    rejected(bd.sparse_fwd, ql, m(1, 8, 15, 64), ck, kp, ix, scale=0.07)
    rejected(bd.sparse_fwd, ql, qp, m(1, 300, 256), kp, ix, scale=0.07)
    rejected(bd.sparse_fwd, ql, qp, ck, m(1, 299, 64), ix, scale=0.07)
    rejected(bd.sparse_fwd, ql, qp, ck, kp, i32(1, 7, 32), scale=0.07)
    rejected(bd.sparse_fwd, ql, qp, ck, kp, ix, scale=0.07, lse=f32(1, 8, 8))
    rejected(bd.sparse_fwd, ql, qp, ck, kp, ix, scale=0.07, out=m(1, 8, 16 * 256))


# ------------------------------------------------------------------ decode
def test_decode_mismatched_tensors():
    q, kv = m(4, 16, 576), m(4, 100, 576)
    rejected(bd.decode_fwd, q, m(4, 100, 512), scale=0.07)                    # cache width
    rejected(bd.decode_fwd, q, m(3, 100, 576), scale=0.07, match="cache slots")
    rejected(bd.decode_fwd, q, kv, scale=0.07, out=m(4, 16, 256))
    rejected(bd.decode_fwd, q, kv, scale=0.07, lse=f32(4, 8))
    rejected(bd.decode_fwd, q, kv, scale=0.07, kv_lens=i32(3))
    rejected(bd.decode_fwd, q, kv, scale=0.07, kv_slots=i32(5))
    rejected(bd.decode_fwd, m(4, 16, 512), m(4, 100, 512), scale=0.07, q_rope=m(4, 16, 64),
             k_rope=m(4, 90, 64))
    rejected(bd.decode_fwd, m(4, 16, 512), m(4, 100, 512), scale=0.07, q_rope=m(4, 16, 64), match="both")


# ------------------------------------------------------------- ring, V-up
def test_ring_mismatched_tensors():
    q = m(1, 4, 256, 576)
    rejected(bd.ring_fwd, q, m(1, 1, 200, 576), 4, scale=0.07)
    rejected(bd.ring_fwd, q, m(1, 2, 256, 576), 4, scale=0.07)
    rejected(bd.ring_fwd, q, m(1, 1, 256, 576), 4, scale=0.07, out=m(1, 4, 255, 512))
    rejected(bd.ring_fwd, q, m(1, 1, 256, 576), 4, scale=0.07, lse=f32(1, 4, 128))


def test_vup_mismatched_tensors():
    rejected(bd.vup, m(1, 4, 10, 512), m(4, 128, 512), out=m(1, 10, 4, 64))
    rejected(bd.vup, m(1, 4, 10, 512), m(3, 128, 512))


def test_debug_gather_mismatched_tensors():
    rejected(bd.debug_gather, m(1, 300, 512), m(1, 299, 64), i32(10))
    rejected(bd.debug_gather, m(1, 300, 512), m(1, 300, 64), i32(10), b=1, match="outside")
