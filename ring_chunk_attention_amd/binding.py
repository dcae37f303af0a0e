"""ctypes binding of libmla355.so.

Argument marshalling only: tensors are checked for dtype/device/layout, turned
into ``mla_rows`` views (pointer + element strides) and handed to the C ABI on
torch's current stream.  Every step of the computation runs in the library's
HIP kernels; there is no fallback.  If the library is missing or cannot be
loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla355.so")

MLA_CAUSAL = 1
MLA_OUT_F32 = 2
MLA_PREV_OUT_F32 = 4
MLA_VALID_LENS = 8
MLA_SEQ_LENS_QK = 16
MLA_OUT_MX4 = 1  # mla_sparse_fwd
MLA_RING_ORDER = 0
MLA_RING_BALANCED = 1
_RING_ORDERS = {"ring": MLA_RING_ORDER, "balanced": MLA_RING_BALANCED}


class MlaRows(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64),
        ("stride_t", ctypes.c_int64),
    ]


_P = ctypes.POINTER(MlaRows)


class MlaFwdCall(ctypes.Structure):
    """mla_fwd_call: the arguments of one shared-latent mla_fwd call."""
    _fields_ = [("q", _P), ("q_rope", _P), ("kv", _P), ("k_rope", _P),
                ("B", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Nq", ctypes.c_int64), ("Nkv", ctypes.c_int64),
                ("dq", ctypes.c_int32), ("dr", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("scale", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("q_offset", ctypes.c_int64), ("kv_offset", ctypes.c_int64),
                ("prev_out", _P), ("prev_lse", _P), ("out", _P), ("lse", _P)]


MAX_GROUP = 4   # MLA_MAX_GROUP


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python ring_chunk_attention_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.mla_fwd.restype = ctypes.c_int
    lib.mla_fwd.argtypes = [
        _P, _P, _P, _P, _P,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_int32,
        ctypes.c_float, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64,
        _P, _P, _P, _P, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_fwd_fp8.restype = ctypes.c_int
    lib.mla_fwd_fp8.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64, _P, _P, ctypes.c_void_p,
                                ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_fwd_group.restype = ctypes.c_int
    lib.mla_fwd_group.argtypes = [ctypes.c_int32, ctypes.POINTER(MlaFwdCall), ctypes.c_void_p]
    lib.mla_merge_lse.restype = ctypes.c_int
    lib.mla_merge_lse.argtypes = [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_int32, _P, _P, ctypes.c_void_p]
    lib.mla_sparse_fwd.restype = ctypes.c_int
    lib.mla_sparse_fwd.argtypes = [_P, _P, _P, _P, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_float, ctypes.c_uint32, _P, _P, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_debug_gather.restype = ctypes.c_int
    lib.mla_debug_gather.argtypes = [_P, _P, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_version.restype = ctypes.c_char_p
    lib.mla_version.argtypes = []
    lib.mla_workspace_size.restype = ctypes.c_size_t
    lib.mla_workspace_size.argtypes = []
    lib.mla_decode_fwd.restype = ctypes.c_int
    lib.mla_decode_fwd.argtypes = [_P, _P, _P, _P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_float, ctypes.c_int32, _P, _P, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_vup.restype = ctypes.c_int
    lib.mla_vup.argtypes = [_P, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                            ctypes.c_int32, ctypes.c_uint32, _P, ctypes.c_void_p]
    lib.mla_decode_fwd_noalloc.restype = ctypes.c_int
    lib.mla_decode_fwd_noalloc.argtypes = [_P, _P, _P, _P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_float, ctypes.c_int32, _P, _P, ctypes.c_void_p]
    lib.mla_decode_workspace_size.restype = ctypes.c_size_t
    lib.mla_decode_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                              ctypes.c_int32]
    lib.mla_ring_fwd.restype = ctypes.c_int
    lib.mla_ring_fwd.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_ring_workspace_size.restype = ctypes.c_size_t
    lib.mla_ring_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
    lib.mla_ring_schedule.restype = ctypes.c_int
    lib.mla_ring_schedule.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                      ctypes.POINTER(ctypes.c_int32)]
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH

EXPORTS = ("mla_fwd", "mla_fwd_fp8", "mla_fwd_group", "mla_merge_lse", "mla_sparse_fwd", "mla_decode_fwd",
           "mla_decode_fwd_noalloc", "mla_vup",
           "mla_debug_gather", "mla_last_error", "mla_version", "mla_workspace_size", "mla_decode_workspace_size",
           "mla_ring_fwd", "mla_ring_workspace_size", "mla_ring_schedule")


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"mla355 status {status}: {message}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        raise MlaError(status, LIB.mla_last_error().decode())


def version() -> str:
    return LIB.mla_version().decode()


# ---------------------------------------------------------------------------
# views
# ---------------------------------------------------------------------------
def _need(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor")


def _shape(t: torch.Tensor, name: str, shape: Tuple[int, ...], device: torch.device) -> None:
    """The library sees only pointers and the sizes passed beside them, so a
    tensor whose shape or device does not match those sizes would be read or
    written out of bounds: such a call is refused here, before the ABI."""
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: expected shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device} (all tensors of a call on one device)")


def _rows_bhtd(t: torch.Tensor, name: str, dtype: torch.dtype = torch.bfloat16) -> MlaRows:
    """[B, H, T, D] (inner dim contiguous) -> view."""
    _need(t, name, dtype)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name}: expected [B, H, T, D] with a contiguous last dim")
    return MlaRows(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _rows_thd(t: torch.Tensor, name: str, dtype: torch.dtype = torch.bfloat16) -> MlaRows:
    """[T, H, D] (tokens outermost) -> view with b = 0."""
    _need(t, name, dtype)
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name}: expected [T, H, D] with a contiguous last dim")
    return MlaRows(t.data_ptr(), 0, t.stride(1), t.stride(0))


def _lse_bht(t: torch.Tensor, name: str) -> MlaRows:
    _need(t, name, torch.float32)
    if t.dim() != 3:
        raise ValueError(f"{name}: expected [B, H, T]")
    return MlaRows(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _lse_ht(t: torch.Tensor, name: str) -> MlaRows:
    _need(t, name, torch.float32)
    if t.dim() != 2:
        raise ValueError(f"{name}: expected [H, T]")
    return MlaRows(t.data_ptr(), 0, t.stride(0), t.stride(1))


def _ref(r: Optional[MlaRows]):
    return ctypes.byref(r) if r is not None else None


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# One workspace per (device, stream): calls on one stream run one after
# another, so they can share it; calls on different streams get their own.
_WORKSPACES = {}


def _workspace(device: torch.device, workspace) -> Tuple[Optional[int], int]:
    """(pointer, bytes) of the workspace for a call on the current stream:
    ``"auto"`` -> this stream's cached one, None -> no workspace (row blocks
    by launch index), a uint8 GPU tensor -> that tensor."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace: expected 'auto', None or a uint8 tensor")
        key = (device.index if device.index is not None else torch.cuda.current_device(),
               torch.cuda.current_stream(device).cuda_stream)
        ws = _WORKSPACES.get(key)
        if ws is None:
            ws = torch.empty(int(LIB.mla_workspace_size()), dtype=torch.uint8, device=device)
            _WORKSPACES[key] = ws
        workspace = ws
    _need(workspace, "workspace", torch.uint8)
    return workspace.data_ptr(), workspace.numel()


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def _fwd_args(q, kv, scale, head_dim_v, causal, q_offset, kv_offset, q_rope, k_rope, v, prev, out,
              lse, want_lse):
    """Views and sizes of one mla_fwd call (outputs allocated if not given)."""
    for t, n in ((q, "q"), (kv, "kv")):
        _need(t, n, torch.bfloat16)
        if t.dim() != 4:
            raise ValueError(f"{n}: expected [B, H, N, D]")
    B, Hq, Nq, dq = q.shape
    Hkv, Nkv = kv.shape[1], kv.shape[2]
    dev_ = q.device
    _shape(kv, "kv", (B, Hkv, Nkv, dq), dev_)
    if (q_rope is None) != (k_rope is None):
        raise ValueError("q_rope and k_rope: give both or neither")
    dr = 0 if q_rope is None else q_rope.shape[-1]
    if q_rope is not None:
        _need(q_rope, "q_rope", torch.bfloat16)
        _need(k_rope, "k_rope", torch.bfloat16)
        _shape(q_rope, "q_rope", (B, Hq, Nq, dr), dev_)
        _shape(k_rope, "k_rope", (B, Hkv, Nkv, dr), dev_)
    dv = head_dim_v if v is None else v.shape[-1]
    if v is not None:
        _need(v, "v", torch.bfloat16)
        _shape(v, "v", (B, Hkv, Nkv, dv), dev_)
    if out is None:
        out = torch.empty((B, Hq, Nq, dv), dtype=torch.bfloat16, device=dev_)
    if lse is None and (want_lse or prev is not None):
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev_)
    _shape(out, "out", (B, Hq, Nq, dv), dev_)
    if lse is not None:
        _shape(lse, "lse", (B, Hq, Nq), dev_)
    if prev is not None:
        if len(prev) != 2:
            raise ValueError("prev: expected (prev_out, prev_lse)")
        _shape(prev[0], "prev_out", (B, Hq, Nq, dv), dev_)
        _shape(prev[1], "prev_lse", (B, Hq, Nq), dev_)
    out_f32 = out.dtype == torch.float32
    prev_f32 = prev is not None and prev[0].dtype == torch.float32
    a = dict(
        q=_rows_bhtd(q, "q"), kv=_rows_bhtd(kv, "kv"),
        out=_rows_bhtd(out, "out", torch.float32 if out_f32 else torch.bfloat16),
        q_rope=_rows_bhtd(q_rope, "q_rope") if q_rope is not None else None,
        k_rope=_rows_bhtd(k_rope, "k_rope") if k_rope is not None else None,
        v=_rows_bhtd(v, "v") if v is not None else None,
        prev_out=(_rows_bhtd(prev[0], "prev_out", torch.float32 if prev_f32 else torch.bfloat16)
                  if prev is not None else None),
        prev_lse=_lse_bht(prev[1], "prev_lse") if prev is not None else None,
        lse=_lse_bht(lse, "lse") if lse is not None else None,
        B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nkv=Nkv, dq=dq, dr=dr, dv=dv, scale=float(scale),
        flags=((MLA_CAUSAL if causal else 0) | (MLA_OUT_F32 if out_f32 else 0)
               | (MLA_PREV_OUT_F32 if prev_f32 else 0)),
        q_offset=q_offset, kv_offset=kv_offset)
    return a, out, lse


def fwd(q: torch.Tensor, kv: torch.Tensor, *, scale: float, head_dim_v: int = 512,
        causal: bool = True, q_offset: int = 0, kv_offset: int = 0,
        q_rope: Optional[torch.Tensor] = None, k_rope: Optional[torch.Tensor] = None,
        v: Optional[torch.Tensor] = None,
        prev: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        want_lse: bool = True, workspace="auto", valid_lens: Optional[torch.Tensor] = None
        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention over [B, H, N, D] tensors (mla_fwd).

    q [B, Hq, Nq, dq], kv [B, Hkv, Nkv, dq]; optional q_rope/k_rope
    [.., dr] and v [B, Hkv, Nkv, dv].  With v None the value is
    kv[..., :head_dim_v].  ``prev = (prev_out, prev_lse)`` folds the result
    into a previous one (out/lse may be the same tensors).  Returns
    (out [B, Hq, Nq, dv] bf16, lse [B, Hq, Nq] fp32 or None).  ``out`` and
    ``prev_out`` may be float32 tensors (a float32 running output for ring
    folds); their dtype selects the flag.  ``workspace``: "auto" (a cached
    per-stream buffer: row blocks from a device queue), None (row blocks by
    launch index) or a uint8 GPU tensor of at least mla_workspace_size()
    bytes.  ``valid_lens`` (int32 [B] on the GPU, shared-latent form): the
    valid rows of each batch of padded tensors (MLA_VALID_LENS); later query
    rows are not written and later key rows not attended.
    """
    a, out, lse = _fwd_args(q, kv, scale, head_dim_v, causal, q_offset, kv_offset, q_rope, k_rope, v,
                            prev, out, lse, want_lse)
    ws, ws_bytes = _workspace(q.device, workspace)
    lens_ptr, flags = None, a["flags"]
    if valid_lens is not None:
        _need(valid_lens, "valid_lens", torch.int32)
        if tuple(valid_lens.shape) != (a["B"],) or not valid_lens.is_contiguous():
            raise ValueError("valid_lens: expected a contiguous [B] tensor")
        if valid_lens.device != q.device:
            raise ValueError(f"valid_lens: on {valid_lens.device}, expected {q.device}")
        lens_ptr, flags = valid_lens.data_ptr(), flags | MLA_VALID_LENS
    _check(LIB.mla_fwd(ctypes.byref(a["q"]), _ref(a["q_rope"]), ctypes.byref(a["kv"]), _ref(a["k_rope"]),
                       _ref(a["v"]), a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"], a["dq"], a["dr"], a["dv"],
                       lens_ptr, a["B"] if lens_ptr else 0, a["scale"], flags, a["q_offset"], a["kv_offset"],
                       _ref(a["prev_out"]), _ref(a["prev_lse"]), ctypes.byref(a["out"]), _ref(a["lse"]),
                       ws, ws_bytes, _stream(q.device)))
    return out, lse


def fwd_fp8(q8: torch.Tensor, kv8: torch.Tensor, *, scale: float, q_scale: float = 1.0, kv_scale: float = 1.0,
            causal: bool = True, q_offset: int = 0, kv_offset: int = 0, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, want_lse: bool = True, workspace="auto"
            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Shared-latent attention over FP8 e4m3 inputs (mla_fwd_fp8): q8
    [B, H, N, 576] and kv8 [B, 1, Nkv, 576] as torch.float8_e4m3fn (or uint8
    codes), dequantised by q_scale and kv_scale.  Returns (out [B, H, N, 512]
    bf16, lse [B, H, N] fp32 or None).  ``workspace`` as for fwd."""
    for t, n in ((q8, "q8"), (kv8, "kv8")):
        if not isinstance(t, torch.Tensor) or t.dtype not in (torch.float8_e4m3fn, torch.uint8):
            raise TypeError(f"{n}: expected a float8_e4m3fn (or uint8 code) tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{n}: must be a GPU tensor")
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{n}: expected [B, H, N, D] with a contiguous last dim")
    B, H, N, dk = q8.shape
    Nkv = kv8.shape[2]
    dev_ = q8.device
    _shape(kv8, "kv8", (B, 1, Nkv, dk), dev_)
    if out is None:
        out = torch.empty((B, H, N, 512), dtype=torch.bfloat16, device=dev_)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev_)
    _shape(out, "out", (B, H, N, 512), dev_)
    if lse is not None:
        _shape(lse, "lse", (B, H, N), dev_)
    vq = MlaRows(q8.data_ptr(), q8.stride(0), q8.stride(1), q8.stride(2))
    vkv = MlaRows(kv8.data_ptr(), kv8.stride(0), kv8.stride(1), kv8.stride(2))
    vo = _rows_bhtd(out, "out")
    vl = _lse_bht(lse, "lse") if lse is not None else None
    ws, ws_bytes = _workspace(dev_, workspace)
    _check(LIB.mla_fwd_fp8(ctypes.byref(vq), ctypes.byref(vkv), B, H, N, Nkv, dk, 512, float(scale),
                           float(q_scale), float(kv_scale), MLA_CAUSAL if causal else 0, int(q_offset),
                           int(kv_offset), ctypes.byref(vo), _ref(vl), ws, ws_bytes, _stream(dev_)))
    return out, lse


def fwd_group(calls) -> list:
    """Up to MAX_GROUP shared-latent fwd calls in one launch (mla_fwd_group).
    ``calls``: a list of dicts of fwd's keyword arguments plus ``q`` and
    ``kv`` (no ``v``, no workspace).  Returns the (out, lse) pair of each."""
    if len(calls) > MAX_GROUP:
        raise ValueError(f"at most {MAX_GROUP} calls per group")
    keep, results = [], []
    arr = (MlaFwdCall * max(1, len(calls)))()
    device = None
    for i, c in enumerate(calls):
        c = dict(c)
        q, kv = c.pop("q"), c.pop("kv")
        device = q.device
        a, out, lse = _fwd_args(q, kv, c.pop("scale"), c.pop("head_dim_v", 512), c.pop("causal", True),
                                c.pop("q_offset", 0), c.pop("kv_offset", 0), c.pop("q_rope", None),
                                c.pop("k_rope", None), None, c.pop("prev", None), c.pop("out", None),
                                c.pop("lse", None), c.pop("want_lse", True))
        if c:
            raise TypeError(f"fwd_group: unexpected arguments {sorted(c)}")
        if a["Hkv"] != 1:
            raise ValueError("fwd_group: shared-latent calls only (one KV head)")
        keep.append(a)
        ref = lambda r: ctypes.pointer(r) if r is not None else None
        arr[i] = MlaFwdCall(ref(a["q"]), ref(a["q_rope"]), ref(a["kv"]), ref(a["k_rope"]), a["B"], a["Hq"],
                            a["Nq"], a["Nkv"], a["dq"], a["dr"], a["dv"], a["scale"], a["flags"],
                            a["q_offset"], a["kv_offset"], ref(a["prev_out"]), ref(a["prev_lse"]),
                            ref(a["out"]), ref(a["lse"]))
        results.append((out, lse))
    if calls:
        _check(LIB.mla_fwd_group(len(calls), arr, _stream(device)))
    return results


def split_fwd(q1: torch.Tensor, q2: torch.Tensor, k1: torch.Tensor, k2: torch.Tensor,
              v: torch.Tensor, *, scale: float, seq_lens: Optional[torch.Tensor] = None,
              causal: bool = True, prev: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
              workspace="auto") -> Tuple[torch.Tensor, torch.Tensor]:
    """Split query/key ring step over [T, H, D] tensors (mla_fwd, Ascend
    RingMLAOperation layout): q1 [T, H, 128], q2 [T, H, 64], k1 [Tk, Hkv, 128],
    k2 [Tk, Hkv, 64], v [Tk, Hkv, 128]; seq_lens int32 on the GPU, [batch]
    (Tk == T: each sequence owns the same tokens of both) or [2, batch]
    (query lengths, then key lengths: MLA_SEQ_LENS_QK); prev = (prev_out
    [T, H, 128], prev_lse [H, T]).  Returns out [T, H, 128] and lse [H, T].
    ``out`` and ``prev_out`` may be float32 tensors (their dtype selects
    MLA_OUT_F32 / MLA_PREV_OUT_F32).  ``workspace`` as for fwd."""
    for t, n in ((q1, "q1"), (q2, "q2"), (k1, "k1"), (k2, "k2"), (v, "v")):
        _need(t, n, torch.bfloat16)
        if t.dim() != 3:
            raise ValueError(f"{n}: expected [T, H, D]")
    T, H, dq = q1.shape
    Tk, Hkv = k1.shape[0], k1.shape[1]
    dr = q2.shape[2]
    dv = v.shape[2]
    dev_ = q1.device
    two_rows = seq_lens is not None and seq_lens.dim() == 2
    if Tk != T and not two_rows:
        raise ValueError(f"k1: {Tk} key tokens, expected {T} (the query tokens) unless seq_lens is [2, batch]")
    _shape(q2, "q2", (T, H, dr), dev_)
    _shape(k1, "k1", (Tk, Hkv, dq), dev_)
    _shape(k2, "k2", (Tk, Hkv, dr), dev_)
    _shape(v, "v", (Tk, Hkv, dv), dev_)
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev_)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=dev_)
    _shape(out, "out", (T, H, dv), dev_)
    _shape(lse, "lse", (H, T), dev_)
    if seq_lens is not None:
        _need(seq_lens, "seq_lens", torch.int32)
        if seq_lens.dim() not in (1, 2) or (two_rows and seq_lens.shape[0] != 2) or not seq_lens.is_contiguous():
            raise ValueError("seq_lens: expected a contiguous [batch] or [2, batch] tensor")
        if seq_lens.device != dev_:
            raise ValueError(f"seq_lens: on {seq_lens.device}, expected {dev_}")
    out_f32 = out.dtype == torch.float32
    prev_f32 = prev is not None and prev[0].dtype == torch.float32
    views = [_rows_thd(q1, "q1"), _rows_thd(q2, "q2"), _rows_thd(k1, "k1"), _rows_thd(k2, "k2"),
             _rows_thd(v, "v")]
    vpo = vpl = None
    if prev is not None:
        if len(prev) != 2:
            raise ValueError("prev: expected (prev_out, prev_lse)")
        _shape(prev[0], "prev_out", (T, H, dv), dev_)
        _shape(prev[1], "prev_lse", (H, T), dev_)
        vpo = _rows_thd(prev[0], "prev_out", torch.float32 if prev_f32 else torch.bfloat16)
        vpl = _lse_ht(prev[1], "prev_lse")
    vout = _rows_thd(out, "out", torch.float32 if out_f32 else torch.bfloat16)
    vl = _lse_ht(lse, "lse")
    flags = ((MLA_CAUSAL if causal else 0) | (MLA_OUT_F32 if out_f32 else 0)
             | (MLA_PREV_OUT_F32 if prev_f32 else 0) | (MLA_SEQ_LENS_QK if two_rows else 0))
    _check(LIB.mla_fwd(ctypes.byref(views[0]), ctypes.byref(views[1]), ctypes.byref(views[2]),
                       ctypes.byref(views[3]), ctypes.byref(views[4]),
                       1, H, Hkv, T, Tk, dq, dr, dv,
                       seq_lens.data_ptr() if seq_lens is not None else None,
                       seq_lens.shape[-1] if seq_lens is not None else 0,
                       float(scale), flags, 0, 0,
                       _ref(vpo), _ref(vpl), ctypes.byref(vout), ctypes.byref(vl),
                       *_workspace(dev_, workspace), _stream(dev_)))
    return out, lse


def merge(out_a: torch.Tensor, lse_a: torch.Tensor, out_b: torch.Tensor, lse_b: torch.Tensor,
          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """LSE merge of two [B, H, N, dv] partial results (mla_merge_lse)."""
    _need(out_a, "out_a", torch.bfloat16)
    if out_a.dim() != 4:
        raise ValueError("out_a: expected [B, H, N, dv]")
    B, H, N, dv = out_a.shape
    dev_ = out_a.device
    if out is None:
        out = torch.empty_like(out_a)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev_)
    for t, n in ((out_b, "out_b"), (out, "out")):
        _shape(t, n, (B, H, N, dv), dev_)
    for t, n in ((lse_a, "lse_a"), (lse_b, "lse_b"), (lse, "lse")):
        _shape(t, n, (B, H, N), dev_)
    va, vb, vo = _rows_bhtd(out_a, "out_a"), _rows_bhtd(out_b, "out_b"), _rows_bhtd(out, "out")
    la, lb, lo = _lse_bht(lse_a, "lse_a"), _lse_bht(lse_b, "lse_b"), _lse_bht(lse, "lse")
    _check(LIB.mla_merge_lse(ctypes.byref(va), ctypes.byref(la), ctypes.byref(vb), ctypes.byref(lb),
                             B, H, N, dv, ctypes.byref(vo), ctypes.byref(lo), _stream(dev_)))
    return out, lse


def sparse_fwd(q_lift: torch.Tensor, q_pe: torch.Tensor, c_kv: torch.Tensor, k_pe: torch.Tensor,
               topk_idx: torch.Tensor, *, scale: float, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True, workspace="auto",
               mx4: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Top-k sparse latent attention (mla_sparse_fwd): q_lift [B,S,H,L],
    q_pe [B,S,H,R], c_kv [B,S_kv,L], k_pe [B,S_kv,R], topk_idx int32
    [B,S,K] -> out [B, S, H*L] bf16 and lse [B, S, H] fp32.  ``workspace`` as
    for fwd.  ``mx4``: each head's columns in MX 4-pack order (MLA_OUT_MX4).
    A float32 ``out`` selects MLA_OUT_F32 (the result before its bf16
    rounding)."""
    for t, n in ((q_lift, "q_lift"), (q_pe, "q_pe")):
        _need(t, n, torch.bfloat16)
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{n}: expected [B, S, H, D] with a contiguous last dim")
    for t, n in ((c_kv, "c_kv"), (k_pe, "k_pe")):
        _need(t, n, torch.bfloat16)
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{n}: expected [B, S_kv, D] with a contiguous last dim")
    B, S, H, L = q_lift.shape
    R = q_pe.shape[3]
    S_kv = c_kv.shape[1]
    dev_ = q_lift.device
    _shape(q_pe, "q_pe", (B, S, H, R), dev_)
    _shape(c_kv, "c_kv", (B, S_kv, L), dev_)
    _shape(k_pe, "k_pe", (B, S_kv, R), dev_)
    _need(topk_idx, "topk_idx", torch.int32)
    if topk_idx.dim() != 3 or not topk_idx.is_contiguous() or tuple(topk_idx.shape[:2]) != (B, S):
        raise ValueError("topk_idx: expected a contiguous [B, S, K] tensor")
    if topk_idx.device != dev_:
        raise ValueError(f"topk_idx: on {topk_idx.device}, expected {dev_}")
    K = topk_idx.shape[2]
    if out is None:
        out = torch.empty((B, S, H * L), dtype=torch.bfloat16, device=dev_)
    if lse is None and want_lse:
        lse = torch.empty((B, S, H), dtype=torch.float32, device=dev_)
    out_f32 = out.dtype == torch.float32
    _need(out, "out", torch.float32 if out_f32 else torch.bfloat16)
    _shape(out, "out", (B, S, H * L), dev_)
    if out.stride(2) != 1:
        raise ValueError("out: expected [B, S, H*L] with a contiguous last dim")
    if lse is not None:
        _shape(lse, "lse", (B, S, H), dev_)
    v_ql = MlaRows(q_lift.data_ptr(), q_lift.stride(0), q_lift.stride(2), q_lift.stride(1))
    v_qp = MlaRows(q_pe.data_ptr(), q_pe.stride(0), q_pe.stride(2), q_pe.stride(1))
    v_ck = MlaRows(c_kv.data_ptr(), c_kv.stride(0), 0, c_kv.stride(1))
    v_kp = MlaRows(k_pe.data_ptr(), k_pe.stride(0), 0, k_pe.stride(1))
    v_o = MlaRows(out.data_ptr(), out.stride(0), L * out.stride(2), out.stride(1))
    v_l = None
    if lse is not None:
        _need(lse, "lse", torch.float32)
        v_l = MlaRows(lse.data_ptr(), lse.stride(0), lse.stride(2), lse.stride(1))
    _check(LIB.mla_sparse_fwd(ctypes.byref(v_ql), ctypes.byref(v_qp), ctypes.byref(v_ck),
                              ctypes.byref(v_kp), topk_idx.data_ptr(), B, S, S_kv, H, L, R, K,
                              float(scale), (MLA_OUT_MX4 if mx4 else 0) | (MLA_OUT_F32 if out_f32 else 0),
                              ctypes.byref(v_o), _ref(v_l),
                              *_workspace(q_lift.device, workspace), _stream(q_lift.device)))
    return out, lse


def vup(o: torch.Tensor, w_uv: torch.Tensor, *, out: Optional[torch.Tensor] = None,
        mx4: bool = False) -> torch.Tensor:
    """V-up projection of the latent attention output (mla_vup): o is a
    [B, H, T, 512] bf16 view (fwd's out; sparse_fwd's out as
    ``out.view(B, S, H, 512).transpose(1, 2)``; decode_fwd's out as
    ``out.unsqueeze(2)``), w_uv bf16 [H, 128, 512] contiguous.  Returns out
    [B, T, H, 128] bf16 (o_proj's input row per token), or writes the given
    ``out`` of that shape.  ``mx4``: o's columns are in MX 4-pack order."""
    _need(o, "o", torch.bfloat16)
    if o.dim() != 4:
        raise ValueError("o: expected [B, H, T, L]")
    B, H, T, L = o.shape
    _need(w_uv, "w_uv", torch.bfloat16)
    if w_uv.dim() != 3 or w_uv.shape[0] != H or w_uv.shape[2] != L or not w_uv.is_contiguous():
        raise ValueError("w_uv: expected a contiguous [H, dvh, L] tensor")
    if w_uv.device != o.device:
        raise ValueError(f"w_uv: on {w_uv.device}, expected {o.device}")
    dvh = w_uv.shape[1]
    if out is None:
        out = torch.empty((B, T, H, dvh), dtype=torch.bfloat16, device=o.device)
    _shape(out, "out", (B, T, H, dvh), o.device)
    vo = _rows_bhtd(out.transpose(1, 2), "out")
    _check(LIB.mla_vup(ctypes.byref(_rows_bhtd(o, "o")), w_uv.data_ptr(), B, H, T, L, dvh,
                       MLA_OUT_MX4 if mx4 else 0, ctypes.byref(vo), _stream(o.device)))
    return out


# Decode workspaces, one per (device, stream), grown to the largest call.
_DECODE_WS = {}


def decode_fwd(q: torch.Tensor, kv: torch.Tensor, *, scale: float,
               kv_lens: Optional[torch.Tensor] = None, kv_slots: Optional[torch.Tensor] = None,
               head_dim_v: int = 512,
               q_rope: Optional[torch.Tensor] = None, k_rope: Optional[torch.Tensor] = None,
               n_splits: int = 0, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True,
               workspace: Optional[torch.Tensor] = None, noalloc: bool = False
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Token generation (mla_decode_fwd): q [B, H, dq] (the newest token of
    each sequence), kv [n_slots, Nkv, dq] (the latent cache), optional q_rope
    [B, H, dr] / k_rope [n_slots, Nkv, dr], kv_lens int32 [B] on the GPU
    (valid rows; None = Nkv), kv_slots int32 [B] on the GPU (the cache slot
    of each sequence; None = slot b).  Returns (out [B, H, dv] bf16, lse [B, H] fp32 or
    None).  n_splits = 0 lets the library split the keys; ``workspace`` (a
    uint8 GPU tensor) defaults to a cached per-stream buffer.  ``noalloc``:
    call mla_decode_fwd_noalloc instead, which takes no workspace (the
    library's static device scratch; ``out``/``lse`` should then be given, so
    that nothing is allocated here either)."""
    if (q_rope is None) != (k_rope is None):
        raise ValueError("q_rope and k_rope: give both or neither")
    for t, n in ((q, "q"), (kv, "kv")) + (((q_rope, "q_rope"), (k_rope, "k_rope")) if q_rope is not None else ()):
        _need(t, n, torch.bfloat16)
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{n}: expected a 3-D tensor with a contiguous last dim")
    B, H, dq = q.shape
    Nkv = kv.shape[1]
    dr = 0 if q_rope is None else q_rope.shape[-1]
    dv = head_dim_v
    dev_ = q.device
    _shape(kv, "kv", (kv.shape[0], Nkv, dq), dev_)
    if kv_slots is None and kv.shape[0] < B and Nkv > 0:
        raise ValueError(f"kv: {kv.shape[0]} cache slots for {B} sequences (sequence b reads slot b)")
    if q_rope is not None:
        _shape(q_rope, "q_rope", (B, H, dr), dev_)
        _shape(k_rope, "k_rope", (kv.shape[0], Nkv, dr), dev_)
    if out is None:
        out = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev_)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev_)
    _need(out, "out", torch.bfloat16)
    _shape(out, "out", (B, H, dv), dev_)
    if lse is not None:
        _shape(lse, "lse", (B, H), dev_)
    for t, n in ((kv_lens, "kv_lens"), (kv_slots, "kv_slots")):
        if t is not None:
            _need(t, n, torch.int32)
            if tuple(t.shape) != (B,) or not t.is_contiguous():
                raise ValueError(f"{n}: expected a contiguous [B] tensor")
            if t.device != dev_:
                raise ValueError(f"{n}: on {t.device}, expected {dev_}")
    n_slots = kv.shape[0] if kv_slots is not None else 0
    vq = MlaRows(q.data_ptr(), q.stride(0), q.stride(1), 0)
    vkv = MlaRows(kv.data_ptr(), kv.stride(0), 0, kv.stride(1))
    vqr = MlaRows(q_rope.data_ptr(), q_rope.stride(0), q_rope.stride(1), 0) if dr else None
    vkr = MlaRows(k_rope.data_ptr(), k_rope.stride(0), 0, k_rope.stride(1)) if dr else None
    vo = MlaRows(out.data_ptr(), out.stride(0), out.stride(1), 0)
    vl = None
    if lse is not None:
        _need(lse, "lse", torch.float32)
        vl = MlaRows(lse.data_ptr(), lse.stride(0), lse.stride(1), 0)
    lens_p = kv_lens.data_ptr() if kv_lens is not None else None
    slots_p = kv_slots.data_ptr() if kv_slots is not None else None
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc: the call takes no workspace")
        _check(LIB.mla_decode_fwd_noalloc(ctypes.byref(vq), _ref(vqr), ctypes.byref(vkv), _ref(vkr), lens_p,
                                          slots_p, n_slots, B, H, Nkv, dq, dr, dv, float(scale), n_splits,
                                          ctypes.byref(vo), _ref(vl), _stream(dev_)))
        return out, lse
    need = int(LIB.mla_decode_workspace_size(B, H, Nkv, n_splits))
    if need == 0:
        raise MlaError(2, f"no key split fits Nkv={Nkv} with n_splits={n_splits}")
    if workspace is None:
        key = (q.device.index if q.device.index is not None else torch.cuda.current_device(),
               torch.cuda.current_stream(q.device).cuda_stream)
        workspace = _DECODE_WS.get(key)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            _DECODE_WS[key] = workspace
    _need(workspace, "workspace", torch.uint8)
    _check(LIB.mla_decode_fwd(ctypes.byref(vq), _ref(vqr), ctypes.byref(vkv), _ref(vkr),
                              lens_p, slots_p, n_slots,
                              B, H, Nkv, dq, dr, dv, float(scale), n_splits,
                              ctypes.byref(vo), _ref(vl), workspace.data_ptr(), workspace.numel(),
                              _stream(q.device)))
    return out, lse


def debug_gather(c_kv: torch.Tensor, k_pe: torch.Tensor, idx: torch.Tensor, b: int = 0) -> torch.Tensor:
    """Rows idx[k] of [c_kv | k_pe] of batch b, gathered by the sparse
    kernel's device tile loader (mla_debug_gather): [K, L + R] bf16."""
    _need(c_kv, "c_kv", torch.bfloat16)
    _need(k_pe, "k_pe", torch.bfloat16)
    _need(idx, "idx", torch.int32)
    if idx.dim() != 1 or not idx.is_contiguous():
        raise ValueError("idx: expected a contiguous 1-D int32 tensor")
    if c_kv.dim() != 3 or k_pe.dim() != 3:
        raise ValueError("c_kv, k_pe: expected [B, S_kv, D]")
    L, R = c_kv.shape[2], k_pe.shape[2]
    _shape(k_pe, "k_pe", (c_kv.shape[0], c_kv.shape[1], R), c_kv.device)
    if idx.device != c_kv.device:
        raise ValueError(f"idx: on {idx.device}, expected {c_kv.device}")
    if not 0 <= b < c_kv.shape[0]:
        raise ValueError(f"b = {b} outside the cache's {c_kv.shape[0]} batches")
    K = idx.numel()
    rows = torch.empty((K, L + R), dtype=torch.bfloat16, device=c_kv.device)
    v_ck = MlaRows(c_kv.data_ptr(), c_kv.stride(0), 0, c_kv.stride(1))
    v_kp = MlaRows(k_pe.data_ptr(), k_pe.stride(0), 0, k_pe.stride(1))
    _check(LIB.mla_debug_gather(ctypes.byref(v_ck), ctypes.byref(v_kp), idx.data_ptr(), b,
                                c_kv.shape[1], L, R, K, rows.data_ptr(), _stream(c_kv.device)))
    return rows


# ---------------------------------------------------------------------------
# one-device ring
# ---------------------------------------------------------------------------
def ring_order(r: int, n_chunks: int) -> Sequence[int]:
    """KV chunks query chunk r visits: step s brings chunk (r - s) mod P; chunks
    after r are wholly in the causal future and are skipped."""
    return [(r - s) % n_chunks for s in range(n_chunks) if (r - s) % n_chunks <= r]


def ring_schedule(n_chunks: int, order: str = "ring") -> List[List[Tuple[int, int]]]:
    """The steps of the ring (mla_ring_schedule): a list of steps, each a
    list of (query chunk r, KV chunk k) calls that a ring of devices would
    run together.  Every pair k <= r appears once; a query chunk has at most
    one call per step, and ring_fwd folds its calls in step order.
    ``order``: "ring" (step s is ring step s: chunk r meets KV chunk
    (r - s) mod P) or "balanced" (the same calls in equally full steps, the
    diagonals last)."""
    if order not in _RING_ORDERS:
        raise ValueError(f"unknown ring schedule {order!r}")
    P = int(n_chunks)
    if P < 1:
        raise ValueError("n_chunks must be >= 1")
    launch_of = (ctypes.c_int32 * (P * (P + 1) // 2))()
    n = ctypes.c_int32(0)
    _check(LIB.mla_ring_schedule(P, _RING_ORDERS[order], launch_of, ctypes.byref(n)))
    launches = [[] for _ in range(n.value)]
    for r in range(P):
        for k in range(r + 1):
            launches[launch_of[r * (r + 1) // 2 + k]].append((r, k))
    return launches


def ring_workspace_size(B: int, H: int, N: int, n_chunks: int) -> int:
    """Bytes of the workspace ring_fwd needs (mla_ring_workspace_size): the
    float32 running results of the chunks and the item queue's counter; 0
    for one chunk or no rows."""
    return int(LIB.mla_ring_workspace_size(int(B), int(H), int(N), int(n_chunks)))


def ring_fwd(q: torch.Tensor, kv: torch.Tensor, n_chunks: int, *, scale: float,
             head_dim_v: int = 512, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None,
             carry: Optional[torch.Tensor] = None,
             order: str = "ring") -> Tuple[torch.Tensor, torch.Tensor]:
    """Causal shared-latent attention of q [B,H,N,576] over kv [B,1,N,576]
    processed as a ring of ``n_chunks`` contiguous chunks on one device
    (mla_ring_fwd): chunks of ceil(N / n_chunks) rows (the last may be
    shorter); query chunk r meets each KV chunk k <= r with global offsets,
    and every call after the first folds into the running result
    (TensorRT-LLM mla.py forward_context_with_chunked_prefill; Ascend
    RingMLAOperation calcType).  One launch runs all the calls; ``order``
    (see ring_schedule) sets the order each chunk's calls fold in: ring
    order by default (each chunk's diagonal first), which measures 1-3%
    faster than the balanced steps in the one-launch form.
    ``carry``: the workspace (the float32 running results between folds and
    the launch's item counter), any contiguous GPU tensor of at least
    ring_workspace_size() bytes (allocated if not given)."""
    if order not in _RING_ORDERS:
        raise ValueError(f"unknown ring schedule {order!r}")
    for t, n in ((q, "q"), (kv, "kv")):
        _need(t, n, torch.bfloat16)
        if t.dim() != 4:
            raise ValueError(f"{n}: expected [B, H, N, D]")
    B, H, N, dq = q.shape
    _shape(kv, "kv", (B, 1, N, dq), q.device)
    if out is None:
        out = torch.empty((B, H, N, head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _shape(out, "out", (B, H, N, head_dim_v), q.device)
    _shape(lse, "lse", (B, H, N), q.device)
    need = int(LIB.mla_ring_workspace_size(B, H, N, n_chunks))
    if carry is None and need:
        carry = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws, ws_bytes = None, 0
    if carry is not None:
        if not carry.is_cuda or not carry.is_contiguous():
            raise ValueError("carry: expected a contiguous GPU tensor")
        if carry.device != q.device:
            raise ValueError(f"carry: on {carry.device}, expected {q.device}")
        ws, ws_bytes = carry.data_ptr(), carry.numel() * carry.element_size()
    vq, vkv = _rows_bhtd(q, "q"), _rows_bhtd(kv, "kv")
    vo, vl = _rows_bhtd(out, "out"), _lse_bht(lse, "lse")
    _check(LIB.mla_ring_fwd(ctypes.byref(vq), ctypes.byref(vkv), B, H, N, dq, head_dim_v, float(scale),
                            int(n_chunks), _RING_ORDERS[order], ctypes.byref(vo), ctypes.byref(vl),
                            ws, ws_bytes, _stream(q.device)))
    return out, lse
