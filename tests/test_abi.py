"""The C ABI: every function include/mla355.h declares is exported by
libmla355.so, and invalid arguments are rejected before anything is launched
(these checks run on the host, so they need no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla355.h")
LIB = os.path.join(ROOT, "ring_chunk_attention_amd", "libmla355.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("mla_fwd", "mla_merge_lse", "mla_sparse_fwd", "mla_debug_gather",
                 "mla_last_error", "mla_version"):
        assert want in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "build the library first: python ring_chunk_attention_amd/build.py"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(mla_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"


def test_binding_exports_list_matches_header():
    from ring_chunk_attention_amd import EXPORTS
    assert sorted(EXPORTS) == declared_functions()


# ---------------------------------------------------------------------------
# validation (host only: these calls fail before touching the GPU)
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def lib():
    from ring_chunk_attention_amd.binding import LIB as L
    return L


class Rows(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64)]


FAKE = 0x10000000  # an aligned address that is never dereferenced: validation fails first


def rows(data=FAKE, sb=128 * 8192 * 576, sh=8192 * 576, st=576):
    return Rows(data, sb, sh, st)


def call_fwd(lib, q=None, kv=None, out=None, lse=None, v=None, q_rope=None, k_rope=None,
             B=1, Hq=128, Hkv=1, Nq=8192, Nkv=8192, dq=576, dr=0, dv=512, seq_lens=None, n_seqs=0,
             scale=0.072, flags=1, q_off=0, kv_off=0, prev_out=None, prev_lse=None,
             workspace=None, workspace_bytes=0):
    from ring_chunk_attention_amd.binding import MlaRows
    def conv(r):
        return None if r is None else ctypes.byref(MlaRows(r.data, r.stride_b, r.stride_h, r.stride_t))
    q = rows() if q is None else q
    kv = rows() if kv is None else kv
    out = rows(st=512) if out is None else out
    return lib.mla_fwd(conv(q), conv(q_rope), conv(kv), conv(k_rope), conv(v), B, Hq, Hkv, Nq, Nkv,
                       dq, dr, dv, seq_lens, n_seqs, scale, flags, q_off, kv_off,
                       conv(prev_out), conv(prev_lse), conv(out), conv(lse), workspace, workspace_bytes,
                       None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(Hq=6, Hkv=4), MLA_ERR_INVALID_ARG, "multiple of Hkv"),
    (dict(Hq=0), MLA_ERR_INVALID_ARG, "sizes"),
    (dict(dv=500), MLA_ERR_INVALID_ARG, "multiples of 8"),
    (dict(flags=32), MLA_ERR_INVALID_ARG, "flag"),
    (dict(flags=17), MLA_ERR_INVALID_ARG, "MLA_SEQ_LENS_QK needs packed seq_lens"),
    (dict(flags=25, seq_lens=FAKE, n_seqs=1), MLA_ERR_INVALID_ARG, "MLA_SEQ_LENS_QK needs packed seq_lens"),
    (dict(flags=17, seq_lens=FAKE, n_seqs=2, Nkv=100), MLA_ERR_UNSUPPORTED, "no kernel"),
    (dict(flags=17, seq_lens=FAKE, n_seqs=2, q_off=3), MLA_ERR_INVALID_ARG, "q_offset == kv_offset == 0"),
    (dict(flags=5), MLA_ERR_INVALID_ARG, "without prev_out"),
    (dict(scale=float("nan")), MLA_ERR_INVALID_ARG, "scale"),
    (dict(q=Rows(FAKE + 2, 0, 576, 576)), MLA_ERR_INVALID_ARG, "aligned"),
    (dict(kv=Rows(FAKE, 0, 576, 577)), MLA_ERR_INVALID_ARG, "multiples of 8"),
    (dict(q_rope=Rows(FAKE, 0, 64, 64), dr=64, dq=512), MLA_ERR_INVALID_ARG, "both"),
    (dict(prev_out=Rows(FAKE, 0, 512, 512)), MLA_ERR_INVALID_ARG, "prev_out and prev_lse"),
    (dict(dv=640, dq=576), MLA_ERR_INVALID_ARG, "head_dim_v"),
    (dict(Hkv=2, Hq=128), MLA_ERR_UNSUPPORTED, "no kernel"),
    (dict(dq=256, dv=256), MLA_ERR_UNSUPPORTED, "no kernel"),
    (dict(seq_lens=FAKE, n_seqs=2, B=2), MLA_ERR_INVALID_ARG, "B == 1"),
    (dict(seq_lens=FAKE, n_seqs=2, Nkv=100), MLA_ERR_INVALID_ARG, "Nq == Nkv"),
    (dict(workspace=FAKE + 8, workspace_bytes=256), MLA_ERR_INVALID_ARG, "16-byte aligned"),
    (dict(workspace=FAKE, workspace_bytes=255), MLA_ERR_INVALID_ARG, "mla_workspace_size"),
])
def test_fwd_rejects_invalid_arguments(lib, kw, code, msg):
    st = call_fwd(lib, **kw)
    assert st == code
    assert msg in lib.mla_last_error().decode()


def test_fwd_rejects_partial_alias(lib):
    o = Rows(FAKE, 0, 512, 512)
    o2 = Rows(FAKE, 0, 512, 1024)
    l = Rows(FAKE + 4096, 0, 8192, 1)
    st = call_fwd(lib, out=o, prev_out=o2, prev_lse=l, lse=l)
    assert st == MLA_ERR_INVALID_ARG and "alias" in lib.mla_last_error().decode()


def test_merge_rejects_bad_dv(lib):
    from ring_chunk_attention_amd.binding import MlaRows
    r = MlaRows(FAKE, 0, 512, 512)
    st = lib.mla_merge_lse(ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), ctypes.byref(r),
                           1, 4, 16, 12, ctypes.byref(r), ctypes.byref(r), None)
    assert st == MLA_ERR_INVALID_ARG


def test_sparse_rejects_unsupported_dims(lib):
    from ring_chunk_attention_amd.binding import MlaRows
    r = MlaRows(FAKE, 0, 512, 512)
    st = lib.mla_sparse_fwd(ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), FAKE,
                            1, 16, 1024, 128, 256, 64, 128, 0.07, 0, ctypes.byref(r), None, None, 0, None)
    assert st == MLA_ERR_UNSUPPORTED
    st = lib.mla_sparse_fwd(ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), FAKE,
                            1, 16, 1024, 256, 512, 64, 128, 0.07, 0, ctypes.byref(r), None, None, 0, None)
    assert st == MLA_ERR_UNSUPPORTED
    st = lib.mla_sparse_fwd(ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), FAKE,
                            1, 16, 1024, 128, 512, 64, 4097, 0.07, 0, ctypes.byref(r), None, None, 0, None)
    assert st == MLA_ERR_UNSUPPORTED and "4096" in lib.mla_last_error().decode()


def test_sparse_rejects_short_workspace(lib):
    from ring_chunk_attention_amd.binding import MlaRows
    r = MlaRows(FAKE, 0, 512, 512)
    st = lib.mla_sparse_fwd(ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), FAKE,
                            1, 16, 1024, 128, 512, 64, 128, 0.07, 0, ctypes.byref(r), None, FAKE, 16, None)
    assert st == MLA_ERR_INVALID_ARG and "workspace" in lib.mla_last_error().decode()


def test_workspace_size(lib):
    assert lib.mla_workspace_size() == 256


def test_binding_raises_with_message(lib):
    from ring_chunk_attention_amd.binding import MlaError, _check
    call_fwd(lib, Hq=6, Hkv=4)
    with pytest.raises(MlaError, match="multiple of Hkv"):
        _check(MLA_ERR_INVALID_ARG)


def call_decode(lib, q=None, kv=None, out=None, lse=None, kv_lens=None, kv_slots=None, n_slots=0, B=4, H=128,
                Nkv=8192, dq=576, dr=0, dv=512, scale=0.072, n_splits=0, workspace=0x20000000,
                workspace_bytes=1 << 40):
    from ring_chunk_attention_amd.binding import MlaRows
    def conv(r):
        return None if r is None else ctypes.byref(MlaRows(r.data, r.stride_b, r.stride_h, r.stride_t))
    q = rows(sb=128 * 576, sh=576, st=0) if q is None else q
    kv = rows(sb=8192 * 576, sh=0, st=576) if kv is None else kv
    out = rows(sb=128 * 512, sh=512, st=0) if out is None else out
    return lib.mla_decode_fwd(conv(q), None, conv(kv), None, kv_lens, kv_slots, n_slots, B, H, Nkv, dq, dr, dv,
                              scale, n_splits,
                              conv(out), conv(lse), workspace, workspace_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(H=0), MLA_ERR_INVALID_ARG, "sizes"),
    (dict(H=129), MLA_ERR_UNSUPPORTED, "128 heads"),
    (dict(dq=512), MLA_ERR_UNSUPPORTED, "576"),
    (dict(dv=256), MLA_ERR_UNSUPPORTED, "576"),
    (dict(scale=float("inf")), MLA_ERR_INVALID_ARG, "scale"),
    (dict(workspace=None), MLA_ERR_INVALID_ARG, "needs a workspace"),
    (dict(workspace=0x20000010), MLA_ERR_INVALID_ARG, "256-byte aligned"),
    (dict(workspace_bytes=1024), MLA_ERR_INVALID_ARG, "mla_decode_workspace_size"),
    (dict(n_splits=2), MLA_ERR_INVALID_ARG, "no split"),          # 4096 rows a split > 2048
    (dict(Nkv=200000), MLA_ERR_UNSUPPORTED, "no split"),          # > 64 splits of 2048
    (dict(kv_lens=FAKE + 2), MLA_ERR_INVALID_ARG, "kv_lens"),
    (dict(kv_slots=FAKE + 2, n_slots=4), MLA_ERR_INVALID_ARG, "kv_slots"),
    (dict(kv_slots=FAKE, n_slots=0), MLA_ERR_INVALID_ARG, "n_slots"),
    (dict(n_slots=3), MLA_ERR_INVALID_ARG, "n_slots"),
])
def test_decode_rejects_invalid_arguments(lib, kw, code, msg):
    assert call_decode(lib, **kw) == code
    assert msg in lib.mla_last_error().decode()


def test_decode_workspace_size(lib):
    # one split: just the queue counter
    assert lib.mla_decode_workspace_size(1, 128, 200, 1) == 256
    # B=64, 8192 rows: 4 splits of 2048 -> LSE 64*4*128*4 B, partials 64*4*128*512*4 B
    assert lib.mla_decode_workspace_size(64, 128, 8192, 0) == 256 + 64 * 4 * 128 * 4 + 64 * 4 * 128 * 512 * 4
    assert lib.mla_decode_workspace_size(4, 128, 8192, 2) == 0      # a split would exceed 2048 rows
    assert lib.mla_decode_workspace_size(4, 128, 200000, 0) == 0    # beyond 64 splits
    # the longest cache with few sequences: the library's choice stops at 64 splits of 2048
    assert lib.mla_decode_workspace_size(2, 128, 131072, 0) == 256 + 2 * 64 * 128 * 4 + 2 * 64 * 128 * 512 * 4


def test_group_rejects_bad_calls(lib):
    from ring_chunk_attention_amd.binding import MlaFwdCall, MlaRows
    q, kv, out = MlaRows(FAKE, 0, 8192 * 576, 576), MlaRows(FAKE, 0, 8192 * 576, 576), MlaRows(FAKE, 0, 8192 * 512, 512)
    good = MlaFwdCall(ctypes.pointer(q), None, ctypes.pointer(kv), None, 1, 16, 1024, 1024, 576, 0, 512, 0.07, 1,
                      0, 0, None, None, ctypes.pointer(out), None)
    bad = MlaFwdCall(ctypes.pointer(q), None, ctypes.pointer(kv), None, 1, 16, 1024, 1024, 576, 0, 500, 0.07, 1,
                     0, 0, None, None, ctypes.pointer(out), None)
    arr = (MlaFwdCall * 5)(good, bad, good, good, good)
    assert lib.mla_fwd_group(5, arr, None) == MLA_ERR_INVALID_ARG
    assert "[0, 4]" in lib.mla_last_error().decode()
    assert lib.mla_fwd_group(2, arr, None) == MLA_ERR_INVALID_ARG
    assert lib.mla_last_error().decode().startswith("call 1:")
    assert lib.mla_fwd_group(0, None, None) == MLA_OK


@pytest.mark.parametrize("kw,code,msg", [
    (dict(flags=9), MLA_ERR_INVALID_ARG, "needs seq_lens"),
    (dict(flags=9, seq_lens=FAKE, n_seqs=3, B=2), MLA_ERR_INVALID_ARG, "n_seqs == B"),
    (dict(flags=9, seq_lens=FAKE + 2, n_seqs=1), MLA_ERR_INVALID_ARG, "aligned"),
])
def test_fwd_valid_lens_rejects(lib, kw, code, msg):
    assert call_fwd(lib, **kw) == code
    assert msg in lib.mla_last_error().decode()


def test_fwd_valid_lens_split_form_unsupported(lib):
    r = rows(sb=0, sh=128, st=32 * 128)
    st = call_fwd(lib, q=r, kv=r, v=r, q_rope=r, k_rope=r, dq=128, dr=64, dv=128, Hq=32, Hkv=32, flags=9,
                  seq_lens=FAKE, n_seqs=1, out=r)
    assert st == MLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("flags,code,msg", [(4, MLA_ERR_INVALID_ARG, "flag"), (6, MLA_ERR_INVALID_ARG, "flag"),
                                            (3, MLA_ERR_UNSUPPORTED, "MX4")])
def test_sparse_rejects_unknown_flags(lib, flags, code, msg):
    """Bits other than MLA_OUT_MX4 and MLA_OUT_F32 are refused, and the two
    are not combined."""
    from ring_chunk_attention_amd.binding import MlaRows
    r = MlaRows(FAKE, 0, 512, 512)
    st = lib.mla_sparse_fwd(ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), ctypes.byref(r), FAKE,
                            1, 16, 1024, 128, 512, 64, 128, 0.07, flags, ctypes.byref(r), None, None, 0, None)
    assert st == code and msg in lib.mla_last_error().decode()


@pytest.mark.parametrize("args,code,msg", [
    (dict(L=256), MLA_ERR_UNSUPPORTED, "L = 512"),
    (dict(dvh=64), MLA_ERR_UNSUPPORTED, "dvh = 128"),
    (dict(flags=2), MLA_ERR_INVALID_ARG, "flag"),
    (dict(H=0), MLA_ERR_INVALID_ARG, "sizes"),
    (dict(w=FAKE + 8), MLA_ERR_INVALID_ARG, "w_uv"),
    (dict(w=None), MLA_ERR_INVALID_ARG, "w_uv"),
])
def test_vup_rejects(lib, args, code, msg):
    from ring_chunk_attention_amd.binding import MlaRows
    a = dict(B=1, H=4, T=64, L=512, dvh=128, flags=0, w=FAKE)
    a.update(args)
    r = MlaRows(FAKE, 0, 512, 512)
    st = lib.mla_vup(ctypes.byref(r), a["w"], a["B"], a["H"], a["T"], a["L"], a["dvh"], a["flags"],
                     ctypes.byref(r), None)
    assert st == code and msg in lib.mla_last_error().decode()


@pytest.mark.parametrize("order", ["ring", "balanced"])
@pytest.mark.parametrize("P", range(1, 10))
def test_ring_schedule_is_a_valid_fold_order(P, order):
    """Host ring driver: every pair k <= r is called once, a query chunk has
    at most one call per launch (its calls fold one after another), and the
    ring order's launch s is ring step s."""
    from ring_chunk_attention_amd import ring_order, ring_schedule
    launches = ring_schedule(P, order)
    seen = [(r, k) for launch in launches for r, k in launch]
    assert sorted(seen) == sorted((r, k) for r in range(P) for k in range(r + 1))
    for launch in launches:
        rs = [r for r, _ in launch]
        assert len(rs) == len(set(rs))
    if order == "ring":
        for s, launch in enumerate(launches):
            assert sorted(launch) == sorted((r, ring_order(r, P)[s]) for r in range(P) if s < r + 1)
    else:
        # the diagonals together, last; the full calls spread evenly over the
        # launches before them
        assert sorted(launches[-1]) == [(r, r) for r in range(P)]
        sizes = [len(l) for l in launches[:-1]]
        assert len(launches) == P
        if sizes:
            assert max(sizes) - min(sizes) <= 1
            assert sum(sizes) == P * (P - 1) // 2


def test_ring_schedule_rejects_unknown_order():
    from ring_chunk_attention_amd import ring_schedule
    with pytest.raises(ValueError):
        ring_schedule(4, "zigzag")


# ---------------------------------------------------------------------------
# empty problems: a view with no rows may be NULL (PyTorch gives an empty
# GPU tensor a NULL data pointer); nothing is launched, so these run on the
# host
# ---------------------------------------------------------------------------
NULL_ROWS = Rows(0, 0, 0, 0)


@pytest.mark.parametrize("kw", [
    dict(Nq=0, q=NULL_ROWS, out=NULL_ROWS),
    dict(B=0, q=NULL_ROWS, kv=NULL_ROWS, out=NULL_ROWS),
    dict(Nq=0, q=NULL_ROWS, out=NULL_ROWS, lse=NULL_ROWS, prev_out=NULL_ROWS, prev_lse=NULL_ROWS, flags=1),
])
def test_fwd_empty_problem_accepts_null_views(lib, kw):
    assert call_fwd(lib, **kw) == MLA_OK, lib.mla_last_error().decode()


def test_fwd_empty_problem_still_checks_shapes(lib):
    # an empty problem of a shape without a kernel is still reported
    assert call_fwd(lib, Nq=0, q=NULL_ROWS, out=NULL_ROWS, Hkv=2) == MLA_ERR_UNSUPPORTED
    # and a NULL view that holds rows is still missing, even where no row would be read
    assert call_fwd(lib, Nq=0, q=NULL_ROWS, out=NULL_ROWS, kv=NULL_ROWS) == MLA_ERR_INVALID_ARG
    assert "kv: missing" in lib.mla_last_error().decode()
    assert call_fwd(lib, Nkv=0, kv=NULL_ROWS, q=NULL_ROWS) == MLA_ERR_INVALID_ARG
    assert "q: missing" in lib.mla_last_error().decode()


def test_merge_sparse_vup_decode_empty_accept_null_views(lib):
    from ring_chunk_attention_amd.binding import MlaRows
    n = MlaRows(0, 0, 0, 0)
    r = MlaRows(FAKE, 0, 512, 512)
    assert lib.mla_merge_lse(ctypes.byref(n), ctypes.byref(n), ctypes.byref(n), ctypes.byref(n),
                             1, 4, 0, 512, ctypes.byref(n), ctypes.byref(n), None) == MLA_OK
    assert lib.mla_merge_lse(ctypes.byref(n), ctypes.byref(n), ctypes.byref(n), ctypes.byref(n),
                             1, 4, 5, 512, ctypes.byref(n), ctypes.byref(n), None) == MLA_ERR_INVALID_ARG
    # sparse: no queries -> the query side and the index list may be NULL
    assert lib.mla_sparse_fwd(ctypes.byref(n), ctypes.byref(n), ctypes.byref(r), ctypes.byref(r), None,
                              1, 0, 1024, 128, 512, 64, 128, 0.07, 0, ctypes.byref(n), None, None, 0,
                              None) == MLA_OK
    # V-up: no rows
    assert lib.mla_vup(ctypes.byref(n), FAKE, 1, 4, 0, 512, 128, 0, ctypes.byref(n), None) == MLA_OK
    # decode: no sequences
    assert call_decode(lib, B=0, q=NULL_ROWS, kv=NULL_ROWS, out=NULL_ROWS) == MLA_OK


def test_generated_qk_chain_is_current():
    """mla_qk_chain.inc is the output of gen_qk_chain.py as it stands."""
    gen = os.path.join(ROOT, "ring_chunk_attention_amd", "csrc", "gen_qk_chain.py")
    r = subprocess.run(["python3", gen, "--check"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


# ---------------------------------------------------------------------------
# native ring driver (mla_ring_fwd, mla_ring_schedule)
# ---------------------------------------------------------------------------
def _balanced_reference(P):
    """The balanced packing restated: each query chunk's full calls, longest
    chains first, go to its r least-filled launches among the first P - 1
    (ties: the earlier), the diagonals last."""
    full = [[] for _ in range(max(P - 1, 0))]
    for r in range(P - 1, 0, -1):
        slots = sorted(sorted(range(P - 1), key=lambda j: (len(full[j]), j))[:r])
        for k, j in enumerate(slots):
            full[j].append((r, k))
    return [l for l in full if l] + [[(r, r) for r in range(P)]]


@pytest.mark.parametrize("P", range(1, 17))
def test_native_balanced_schedule_matches_its_rule(P):
    from ring_chunk_attention_amd import ring_schedule
    got = [sorted(l) for l in ring_schedule(P, "balanced")]
    want = [sorted(l) for l in _balanced_reference(P)]
    assert got == want


def call_ring(lib, q=None, kv=None, out=None, lse=None, B=1, H=16, N=4096, dq=576, dv=512, scale=0.072,
              n_chunks=4, order=1, workspace=0x20000000, workspace_bytes=1 << 40):
    from ring_chunk_attention_amd.binding import MlaRows
    def conv(r):
        return None if r is None else ctypes.byref(MlaRows(r.data, r.stride_b, r.stride_h, r.stride_t))
    q = rows() if q is None else q
    kv = rows() if kv is None else kv
    out = rows(st=512) if out is None else out
    lse = Rows(FAKE, 0, 4096, 1) if lse is None else lse
    return lib.mla_ring_fwd(conv(q), conv(kv), B, H, N, dq, dv, scale, n_chunks, order, conv(out), conv(lse),
                            workspace, workspace_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n_chunks=0), MLA_ERR_INVALID_ARG, "n_chunks"),
    (dict(n_chunks=65), MLA_ERR_INVALID_ARG, "n_chunks"),
    (dict(order=2), MLA_ERR_INVALID_ARG, "order"),
    (dict(dq=512), MLA_ERR_UNSUPPORTED, "dq = 576"),
    (dict(H=0), MLA_ERR_INVALID_ARG, "sizes"),
    (dict(workspace=None), MLA_ERR_INVALID_ARG, "needs a workspace"),
    (dict(workspace=0x20000010), MLA_ERR_INVALID_ARG, "256-byte aligned"),
    (dict(workspace_bytes=1024), MLA_ERR_INVALID_ARG, "mla_ring_workspace_size"),
    (dict(scale=float("nan")), MLA_ERR_INVALID_ARG, "scale"),        # from the first call's checks
    (dict(q=Rows(FAKE + 2, 0, 576, 576)), MLA_ERR_INVALID_ARG, "aligned"),
])
def test_ring_rejects_invalid_arguments(lib, kw, code, msg):
    assert call_ring(lib, **kw) == code
    assert msg in lib.mla_last_error().decode()


def test_ring_workspace_size_and_empty_ring(lib):
    # the float32 carry, then 256 bytes for the item queue's counter
    assert lib.mla_ring_workspace_size(1, 16, 4096, 4) == 16 * 4096 * 512 * 4 + 256
    assert lib.mla_ring_workspace_size(1, 16, 4096, 1) == 0
    # a ragged length: chunks of ceil(4095 / 4) = 1024 rows, the last 1023
    assert lib.mla_ring_workspace_size(1, 16, 4095, 4) == 16 * 4 * 1024 * 512 * 4 + 256
    # no rows: nothing is launched, and every view may be NULL
    assert call_ring(lib, N=0, q=NULL_ROWS, kv=NULL_ROWS, out=NULL_ROWS, lse=NULL_ROWS, workspace=None,
                     workspace_bytes=0) == MLA_OK


def test_ring_schedule_rejects(lib):
    arr = (ctypes.c_int32 * 10)()
    n = ctypes.c_int32(0)
    assert lib.mla_ring_schedule(4, 7, arr, ctypes.byref(n)) == MLA_ERR_INVALID_ARG
    assert lib.mla_ring_schedule(0, 1, arr, ctypes.byref(n)) == MLA_ERR_INVALID_ARG
    assert lib.mla_ring_schedule(4, 1, None, ctypes.byref(n)) == MLA_ERR_INVALID_ARG
    assert lib.mla_ring_schedule(4, 1, arr, ctypes.byref(n)) == MLA_OK and n.value == 4


def test_sizes_whose_products_overflow_are_rejected(lib):
    """Row counts near the int64 range make the grid and workspace products
    wrap; validation must still refuse them rather than pass a wrapped size."""
    from ring_chunk_attention_amd.binding import MlaRows
    big = 1 << 62
    assert lib.mla_ring_workspace_size(1 << 30, 1 << 30, big, 2) == (1 << 64) - 1
    assert call_ring(lib, N=big, workspace_bytes=1 << 40) == MLA_ERR_UNSUPPORTED
    assert "overflows" in lib.mla_last_error().decode()
    st = call_fwd(lib, B=1 << 30, Nq=big, Nkv=big, lse=Rows(FAKE + (1 << 20), 0, 0, 1))
    assert st == MLA_ERR_UNSUPPORTED and "too large" in lib.mla_last_error().decode()
    a, b, o = (MlaRows(FAKE + i * (1 << 24), 0, 512, 512) for i in range(3))
    la, lb, lo = (MlaRows(FAKE + (3 + i) * (1 << 24), 0, 0, 1) for i in range(3))
    st = lib.mla_merge_lse(ctypes.byref(a), ctypes.byref(la), ctypes.byref(b), ctypes.byref(lb),
                           1 << 30, 128, big, 512, ctypes.byref(o), ctypes.byref(lo), None)
    assert st == MLA_ERR_UNSUPPORTED and "too large" in lib.mla_last_error().decode()


@pytest.mark.parametrize("B,S,S_kv,msg", [(1 << 30, 1 << 40, 1024, "too large"),
                                          (1, 16, 1 << 62, "2 GiB")])
def test_sparse_sizes_whose_products_overflow_are_rejected(lib, B, S, S_kv, msg):
    from ring_chunk_attention_amd.binding import MlaRows
    q, qp, ckv, kpe, o = (MlaRows(FAKE + i * (1 << 24), 0, 512, 512) for i in range(5))
    st = lib.mla_sparse_fwd(ctypes.byref(q), ctypes.byref(qp), ctypes.byref(ckv), ctypes.byref(kpe), FAKE,
                            B, S, S_kv, 128, 512, 64, 128, 0.07, 0, ctypes.byref(o), None, None, 0, None)
    assert st == MLA_ERR_UNSUPPORTED and msg in lib.mla_last_error().decode()


def test_decode_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """64 sequences of 131,072 rows need 64 ranges each: 4096 partial results
    per head, far past the static scratch.  Refused on the host with a
    message naming the scratch, before any device call."""
    from ring_chunk_attention_amd.binding import MlaRows
    q = MlaRows(FAKE, 128 * 576, 576, 0)
    kv = MlaRows(FAKE, 131072 * 576, 0, 576)
    out = MlaRows(FAKE, 128 * 512, 512, 0)
    st = lib.mla_decode_fwd_noalloc(ctypes.byref(q), None, ctypes.byref(kv), None, None, None, 0,
                                    64, 128, 131072, 576, 0, 512, 0.072, 0, ctypes.byref(out), None, None)
    assert st == MLA_ERR_UNSUPPORTED
    msg = lib.mla_last_error().decode()
    assert "scratch" in msg and "83886080" in msg, msg
    # the same sizes with a caller's workspace are a matter of workspace size only
    need = lib.mla_decode_workspace_size(64, 128, 131072, 0)
    assert need > 83886080
