"""Python binding of the ck_decode_attn C ABI (argument marshalling only).

Every step of the attention runs in the HIP kernels of
``libck_decode_attn.so``; torch only supplies device memory and the current
stream.  There is no fallback: if the library is missing, importing the
entry points raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libck_decode_attn.so")

CK_DT_F32 = 0
CK_DT_BF16 = 1
CK_MAX_NQ = 6
CK_MAX_SPLITS = 256
CK_PATH_GATHER = 0
CK_PATH_SCAN = 1
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape", -3: "misaligned pointer",
          -4: "workspace missing or too small", -5: "HIP runtime error",
          -6: "shape needs more than the no-alloc scratch holds"}
EXPORTS = ("ck_decode_attn", "ck_decode_attn_noalloc", "ck_decode_attn_gather", "ck_decode_attn_steps", "ck_decode_attn_q8",
           "ck_kv_append_q8", "ck_decode_attn_workspace_size",
           "ck_decode_attn_plan", "ck_decode_sparse_path", "ck_decode_topk", "ck_decode_topk_plan",
           "ck_decode_topk_workspace_size", "ck_workspace_status", "ck_set_spin_limit", "ck_set_contraction",
           "ck_set_phase_stamps", "ck_status_string")
CK_WS_ERR_MERGE = 1
CK_WS_ERR_TOPK = 2
CONTRACTIONS = {"mfma": 0, "valu": 1, "valu_f32": 2}


class CkError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n_q", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("cap", ctypes.c_int32)]


class Q8CacheC(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("page_tokens", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("units", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("split_target", ctypes.c_int32), ("chunk_min", ctypes.c_int32),
                ("chunk_max", ctypes.c_int32),
                ("granule", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("row_groups", ctypes.c_int32), ("rows_per_group", ctypes.c_int32),
                ("slices", ctypes.c_int32), ("tile", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run decode_attention_flash_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sp = ctypes.POINTER(Shape)
        L.ck_decode_attn_plan.argtypes = [sp, i32, ctypes.c_int, ctypes.c_int, ctypes.POINTER(Plan)]
        L.ck_decode_attn_plan.restype = ctypes.c_int
        L.ck_decode_attn_workspace_size.argtypes = [sp, i32, ctypes.c_int, ctypes.POINTER(sz)]
        L.ck_decode_attn_workspace_size.restype = ctypes.c_int
        L.ck_decode_attn.argtypes = [sp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_int, vp, vp,
                                     ctypes.c_int, vp, vp, sz, ctypes.c_int, vp]
        L.ck_decode_attn.restype = ctypes.c_int
        L.ck_decode_attn_noalloc.argtypes = [sp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_int, vp, vp,
                                             ctypes.c_int, vp, ctypes.c_int, vp]
        L.ck_decode_attn_noalloc.restype = ctypes.c_int
        L.ck_decode_attn_gather.argtypes = [sp, vp, vp, vp, vp, vp, i32, i64, ctypes.c_float,
                                            ctypes.c_int, vp, ctypes.c_int, vp, vp, sz,
                                            ctypes.c_int, vp]
        L.ck_decode_attn_gather.restype = ctypes.c_int
        L.ck_decode_attn_steps.argtypes = [sp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, ctypes.c_int,
                                           vp, vp, sz, ctypes.c_int, vp]
        L.ck_decode_attn_steps.restype = ctypes.c_int
        qp = ctypes.POINTER(Q8CacheC)
        L.ck_decode_attn_q8.argtypes = [sp, vp, qp, vp, ctypes.c_float, ctypes.c_int, vp, ctypes.c_int, vp,
                                        vp, sz, ctypes.c_int, vp]
        L.ck_decode_attn_q8.restype = ctypes.c_int
        L.ck_kv_append_q8.argtypes = [sp, vp, vp, vp, qp, vp]
        L.ck_kv_append_q8.restype = ctypes.c_int
        L.ck_decode_sparse_path.argtypes = [sp, i32, i64, ctypes.POINTER(i32)]
        L.ck_decode_sparse_path.restype = ctypes.c_int
        L.ck_decode_topk.argtypes = [sp, vp, i32, vp, i32, i32, ctypes.c_int, vp, vp, sz, vp]
        L.ck_decode_topk.restype = ctypes.c_int
        L.ck_decode_topk_plan.argtypes = [sp, i32, i32, i32, ctypes.c_int, ctypes.POINTER(i32),
                                          ctypes.POINTER(sz)]
        L.ck_decode_topk_plan.restype = ctypes.c_int
        L.ck_decode_topk_workspace_size.argtypes = [sp, i32, i32, i32, ctypes.POINTER(sz)]
        L.ck_decode_topk_workspace_size.restype = ctypes.c_int
        L.ck_workspace_status.argtypes = [vp, vp, ctypes.POINTER(i32)]
        L.ck_workspace_status.restype = ctypes.c_int
        L.ck_set_spin_limit.argtypes = [i32]
        L.ck_set_spin_limit.restype = ctypes.c_int
        L.ck_set_contraction.argtypes = [i32]
        L.ck_set_contraction.restype = ctypes.c_int
        L.ck_set_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        L.ck_set_phase_stamps.restype = ctypes.c_int
        L.ck_status_string.argtypes = [ctypes.c_int]
        L.ck_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def shape_of(q: torch.Tensor, k_cache: torch.Tensor) -> Shape:
    B, n_q, Hq, D = q.shape
    Bk, cap, Hkv, Dk = k_cache.shape
    if Bk != B or Dk != D:
        raise ValueError(f"q {tuple(q.shape)} and k_cache {tuple(k_cache.shape)} disagree")
    return Shape(B, n_q, Hq, Hkv, D, cap)


def plan(shape: Shape, W: int = 0, num_splits: int = 0, num_cus: int | None = None) -> dict:
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    p = Plan()
    st = lib().ck_decode_attn_plan(ctypes.byref(shape), W, num_splits, num_cus, ctypes.byref(p))
    if st != 0:
        raise CkError(st, "ck_decode_attn_plan")
    return p.as_dict()


def workspace_size(shape: Shape, W: int = 0, num_splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    st = lib().ck_decode_attn_workspace_size(ctypes.byref(shape), W, num_splits, ctypes.byref(n))
    if st != 0:
        raise CkError(st, "ck_decode_attn_workspace_size")
    return n.value


def new_workspace(shape: Shape, W: int = 0, num_splits: int = 0, device=None) -> torch.Tensor | None:
    """A zeroed workspace for this plan (None when none is needed).  Keep one
    per stream and plan: every launch leaves it ready for the next launch of
    the same plan, so it can be reused and captured without a memset, but
    another plan needs its own (or a re-zeroed) one."""
    n = workspace_size(shape, W, num_splits)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device or torch.cuda.current_device())


_ws_cache: dict = {}


def _stream_handle(stream, device) -> int:
    return stream if stream is not None else torch.cuda.current_stream(device).cuda_stream


def _cached_workspace(shape: Shape, W: int, num_splits: int, device, stream_handle) -> torch.Tensor | None:
    n = workspace_size(shape, W, num_splits)
    if n == 0:
        return None
    # A workspace belongs to one plan (its counters are laid out for it) and
    # to one stream (launches that may overlap need different workspaces).
    # Graphs captured without an explicit workspace all record the one of
    # their capture stream: replay such graphs one after another on one
    # stream, or give each graph that may run concurrently its own workspace.
    key = (torch.device(device).index, int(stream_handle or 0),
           tuple(getattr(shape, f) for f, _ in Shape._fields_), W, num_splits)
    ws = _ws_cache.get(key)
    if ws is None:
        ws = torch.zeros(n, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def workspace_status(workspace: torch.Tensor, stream=None) -> int:
    """The sticky status bits of a workspace (``ck_workspace_status``):
    CK_WS_ERR_MERGE when a split merge gave up waiting, CK_WS_ERR_TOPK when a
    top-k row barrier did; 0 when every launch since the buffer was zeroed
    completed its waits.  Synchronizes the stream."""
    v = ctypes.c_int32(0)
    st = lib().ck_workspace_status(_ptr(workspace), ctypes.c_void_p(_stream_handle(stream, workspace.device)),
                                   ctypes.byref(v))
    if st != 0:
        raise CkError(st, "ck_workspace_status")
    return v.value


def set_spin_limit(polls: int) -> None:
    """Polls a bounded wait makes before giving up (``ck_set_spin_limit``;
    0 restores the default).  For tests of the failure path."""
    st = lib().ck_set_spin_limit(int(polls))
    if st != 0:
        raise CkError(st, "ck_set_spin_limit")


def set_contraction(kind: str) -> None:
    """Contraction for plans of up to 8 packed rows (``ck_set_contraction``):
    "mfma" (the default), "valu" (v_dot2 on bf16 pairs) or "valu_f32".
    Process-wide."""
    if kind not in CONTRACTIONS:
        raise ValueError(f"contraction must be one of {sorted(CONTRACTIONS)}")
    st = lib().ck_set_contraction(CONTRACTIONS[kind])
    if st != 0:
        raise CkError(st, "ck_set_contraction")


_stamps_ref = None  # the buffer set with set_phase_stamps, kept alive while set


def set_phase_stamps(stamps) -> None:
    """Phase timestamps of the attention kernels (``ck_set_phase_stamps``):
    a device int64 tensor of workgroups x 16 words, or None to stop.  The
    tensor is held here until stamping is turned off (launches write to it;
    graphs captured while it was set keep writing to it when replayed)."""
    global _stamps_ref
    if stamps is None:
        st = lib().ck_set_phase_stamps(None, 0)
        if st == 0:
            _stamps_ref = None
    else:
        if stamps.dtype != torch.int64 or stamps.dim() != 2 or stamps.shape[1] != 16 or not stamps.is_cuda:
            raise ValueError("stamps must be a device int64 tensor of shape [workgroups, 16]")
        if not stamps.is_contiguous():
            raise ValueError("stamps must be contiguous")
        st = lib().ck_set_phase_stamps(ctypes.c_void_p(stamps.data_ptr()), stamps.shape[0])
        if st == 0:
            _stamps_ref = stamps
    if st != 0:
        raise CkError(st, "ck_set_phase_stamps")


def cached_workspaces() -> list:
    """The workspaces the entry points allocated for themselves."""
    return list(_ws_cache.values()) + list(_topk_ws.values())


def release_workspaces() -> None:
    """Drop the workspaces the entry points allocated for themselves (one
    per device, stream and plan when no ``workspace`` is passed), e.g. after
    the batch shapes in use have changed.  The next call allocates a fresh
    zeroed one.  Graphs captured with a dropped workspace still point at its
    memory: release them first."""
    _ws_cache.clear()
    _topk_ws.clear()


def _check(t: torch.Tensor, name: str, dtype) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _outputs(q, out_dtype, out, lse, return_lse):
    """Checks (or allocates) out [B, n_q, Hq, D] and lse [B, n_q, Hq]: the
    kernels size their stores from q's shape."""
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    else:
        _check(out, "out", out_dtype)
        _check_shape(out, "out", q.shape)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check(lse, "lse", torch.float32)
        _check_shape(lse, "lse", q.shape[:3])
    return out, lse


def _check_lens(kv_lens: torch.Tensor, B: int, name: str = "kv_lens") -> None:
    _check(kv_lens, name, torch.int32)
    if kv_lens.dim() != 1 or kv_lens.numel() != B:
        raise ValueError(f"{name} must have shape ({B},), got {tuple(kv_lens.shape)}")


def _prepare(q, k_cache, v_cache, kv_lens, out_dtype, out, lse, return_lse):
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    _check(q, "q", torch.bfloat16)
    _check(k_cache, "k_cache", torch.bfloat16)
    _check(v_cache, "v_cache", torch.bfloat16)
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [B, n_q, Hq, D] and k_cache [B, cap, Hkv, D]")
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    shape = shape_of(q, k_cache)
    _check_lens(kv_lens, shape.B)
    out, lse = _outputs(q, out_dtype, out, lse, return_lse)
    odt = CK_DT_BF16 if out_dtype == torch.bfloat16 else CK_DT_F32
    return shape, out, lse, odt


def decode_attn(q, k_cache, v_cache, kv_lens, *, scale: float | None = None, causal: bool = False,
                keep_mask=None, out_dtype=torch.float32, out=None, lse=None, return_lse=False,
                workspace=None, num_splits: int = 0, stream=None):
    """Dense length-aware decode attention (``ck_decode_attn``).

    q [B, n_q, Hq, D] bf16, k_cache / v_cache [B, cap, Hkv, D] bf16,
    kv_lens [B] int32 (device), keep_mask [B, n_q, Hkv, cap] uint8 or None.
    Returns out (and lse [B, n_q, Hq] fp32 when return_lse or lse is given).
    """
    shape, out, lse, odt = _prepare(q, k_cache, v_cache, kv_lens, out_dtype, out, lse, return_lse)
    if keep_mask is not None:
        _check(keep_mask, "keep_mask", torch.uint8)
        _check_shape(keep_mask, "keep_mask", (shape.B, shape.n_q, shape.Hkv, shape.cap))
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    st_handle = _stream_handle(stream, q.device)
    if workspace is None:
        workspace = _cached_workspace(shape, 0, num_splits, q.device, st_handle)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ck_decode_attn(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(kv_lens), ctypes.c_float(scale), 1 if causal else 0,
                              _ptr(keep_mask), _ptr(out), odt, _ptr(lse), _ptr(workspace),
                              ws_bytes, num_splits, ctypes.c_void_p(st_handle))
    if st != 0:
        raise CkError(st, "ck_decode_attn")
    return (out, lse) if (return_lse or lse is not None) else out


def decode_attn_noalloc(q, k_cache, v_cache, kv_lens, *, scale: float | None = None, causal: bool = False,
                        keep_mask=None, out_dtype=torch.float32, out=None, lse=None, return_lse=False,
                        num_splits: int = 0, stream=None):
    """``decode_attn`` through ``ck_decode_attn_noalloc``: the split merge
    uses the library's fixed per-device scratch, so the launch needs no
    workspace (the outputs are still the caller's).  Calls that may overlap
    on one device must not be issued."""
    shape, out, lse, odt = _prepare(q, k_cache, v_cache, kv_lens, out_dtype, out, lse, return_lse)
    if keep_mask is not None:
        _check(keep_mask, "keep_mask", torch.uint8)
        _check_shape(keep_mask, "keep_mask", (shape.B, shape.n_q, shape.Hkv, shape.cap))
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    st_handle = _stream_handle(stream, q.device)
    st = lib().ck_decode_attn_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens),
                                      ctypes.c_float(scale), 1 if causal else 0, _ptr(keep_mask), _ptr(out), odt,
                                      _ptr(lse), num_splits, ctypes.c_void_p(st_handle))
    if st != 0:
        raise CkError(st, "ck_decode_attn_noalloc")
    return (out, lse) if (return_lse or lse is not None) else out


def decode_attn_gather(q, k_cache, v_cache, kv_lens, idx, *, scale: float | None = None,
                       causal: bool = False, out_dtype=torch.float32, out=None, lse=None,
                       return_lse=False, workspace=None, num_splits: int = 0, stream=None):
    """Gathered decode attention over per-query index lists
    (``ck_decode_attn_gather``).  idx is int32 [B, n_q, Hkv, W] (one list per
    query and KV head) or [B, n_q, W] (one list per query, shared by heads)."""
    shape, out, lse, odt = _prepare(q, k_cache, v_cache, kv_lens, out_dtype, out, lse, return_lse)
    _check(idx, "idx", torch.int32)
    if idx.dim() == 4:
        if tuple(idx.shape[:3]) != (shape.B, shape.n_q, shape.Hkv):
            raise ValueError("idx must be [B, n_q, Hkv, W]")
        W = idx.shape[3]
        head_stride = W
    elif idx.dim() == 3:
        if tuple(idx.shape[:2]) != (shape.B, shape.n_q):
            raise ValueError("shared idx must be [B, n_q, W]")
        W = idx.shape[2]
        head_stride = 0
    else:
        raise ValueError("idx must be 3-D or 4-D")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    st_handle = _stream_handle(stream, q.device)
    if workspace is None:
        workspace = _cached_workspace(shape, W, num_splits, q.device, st_handle)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ck_decode_attn_gather(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(kv_lens), _ptr(idx), W, head_stride,
                                     ctypes.c_float(scale), 1 if causal else 0, _ptr(out), odt,
                                     _ptr(lse), _ptr(workspace), ws_bytes, num_splits,
                                     ctypes.c_void_p(st_handle))
    if st != 0:
        raise CkError(st, "ck_decode_attn_gather")
    return (out, lse) if (return_lse or lse is not None) else out


def sparse_path(shape: Shape, W: int, n_kv: int) -> str:
    """"gather" or "scan": the faster entry point for a top-k selection of W
    cells per query over lengths up to n_kv (``ck_decode_sparse_path``)."""
    path = ctypes.c_int32(-1)
    st = lib().ck_decode_sparse_path(ctypes.byref(shape), int(W), int(n_kv), ctypes.byref(path))
    if st != 0:
        raise CkError(st, "ck_decode_sparse_path")
    return "scan" if path.value == CK_PATH_SCAN else "gather"


def decode_attn_sparse(q, k_cache, v_cache, kv_lens, idx, *, keep_mask=None, n_kv: int | None = None,
                       scale: float | None = None, causal: bool = False, out_dtype=torch.float32, out=None,
                       lse=None, return_lse=False, num_splits: int = 0, stream=None):
    """Attention over a top-k selection given as index lists ``idx`` (and,
    optionally, the same cells as ``keep_mask``): runs the gather or the
    masked scan, whichever ``sparse_path`` names for the shape, W and n_kv
    (default: the cache capacity).  The scan needs the mask; without one the
    gather runs.  Workspaces come from the per-plan cache."""
    shape = shape_of(q, k_cache)
    W = idx.shape[-1]
    path = sparse_path(shape, W, shape.cap if n_kv is None else n_kv)
    kw = dict(scale=scale, causal=causal, out_dtype=out_dtype, out=out, lse=lse, return_lse=return_lse,
              num_splits=num_splits, stream=stream)
    if path == "scan" and keep_mask is not None:
        return decode_attn(q, k_cache, v_cache, kv_lens, keep_mask=keep_mask, **kw)
    return decode_attn_gather(q, k_cache, v_cache, kv_lens, idx, **kw)


def _topk_shape(scores: torch.Tensor, num_kv_heads: int | None) -> tuple[Shape, int]:
    if scores.dim() != 4:
        raise ValueError("scores must be [B, n_q, Hs, cap]")
    B, n_q, Hs, cap = scores.shape
    Hkv = Hs if num_kv_heads is None else int(num_kv_heads)
    # Hq and D do not enter the selection; the shape carries placeholders.
    return Shape(B, n_q, Hkv, Hkv, 128, cap), Hs


def topk_plan(scores_shape, k: int, tail: int = 0, num_kv_heads: int | None = None,
              num_cus: int | None = None) -> dict:
    """Workgroups per row and workspace bytes of ``ck_decode_topk`` for scores
    of shape [B, n_q, Hs, cap] (``ck_decode_topk_plan``)."""
    B, n_q, Hs, cap = scores_shape
    Hkv = Hs if num_kv_heads is None else int(num_kv_heads)
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    P, n = ctypes.c_int32(0), ctypes.c_size_t(0)
    st = lib().ck_decode_topk_plan(ctypes.byref(Shape(B, n_q, Hkv, Hkv, 128, cap)), Hs, k, tail, num_cus,
                                   ctypes.byref(P), ctypes.byref(n))
    if st != 0:
        raise CkError(st, "ck_decode_topk_plan")
    return {"wgs_per_row": P.value, "workspace_bytes": n.value}


_topk_ws = {}


def decode_topk(scores, kv_lens, k: int, *, tail: int = 0, causal: bool = False, num_kv_heads: int | None = None,
                out=None, workspace=None, stream=None):
    """Top-k index lists (``ck_decode_topk``): for each (sequence, query, score
    head) row of scores [B, n_q, Hs, cap] fp32, the k highest-scoring cells
    before the window's last ``tail`` cells, then those tail cells, ascending,
    padded with -1: int32 [B, n_q, Hs, k + tail], ready for decode_attn_gather
    (Hs = 1 gives one list per query: pass it as [B, n_q, W])."""
    _check(scores, "scores", torch.float32)
    shape, Hs = _topk_shape(scores, num_kv_heads)
    _check_lens(kv_lens, shape.B)
    W = int(k) + int(tail)
    if out is None:
        out = torch.empty((shape.B, shape.n_q, Hs, W), dtype=torch.int32, device=scores.device)
    _check(out, "out", torch.int32)
    if tuple(out.shape) != (shape.B, shape.n_q, Hs, W):
        raise ValueError("out must be [B, n_q, Hs, k + tail]")
    st_handle = _stream_handle(stream, scores.device)
    if workspace is None:
        n = ctypes.c_size_t(0)
        st = lib().ck_decode_topk_workspace_size(ctypes.byref(shape), Hs, int(k), int(tail), ctypes.byref(n))
        if st != 0:
            raise CkError(st, "ck_decode_topk_workspace_size")
        if n.value:
            # Every launch leaves the workspace zeroed, so any plan may reuse
            # it afterwards; launches on different streams may overlap and
            # get their own.
            key = (n.value, scores.device, int(st_handle or 0))
            if key not in _topk_ws:
                _topk_ws[key] = torch.zeros(n.value, dtype=torch.uint8, device=scores.device)
            workspace = _topk_ws[key]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ck_decode_topk(ctypes.byref(shape), _ptr(scores), Hs, _ptr(kv_lens), int(k), int(tail),
                              1 if causal else 0, _ptr(out), _ptr(workspace), ws_bytes, ctypes.c_void_p(st_handle))
    if st != 0:
        raise CkError(st, "ck_decode_topk")
    return out


def decode_attn_steps(q, k_cache, v_cache, kv_lens, k_step, v_step, *, scale: float | None = None,
                      out_dtype=torch.float32, out=None, lse=None, return_lse=False, workspace=None,
                      num_splits: int = 0, stream=None):
    """Verification queries over the cache prefix plus their own step rows
    (``ck_decode_attn_steps``): query i sees cache cells j < kv_lens[b] and
    step rows 0..i of k_step / v_step [B, n_q, Hkv, D] bf16, which are not in
    the cache.  Same result as ``decode_attn(..., causal=True)`` over a cache
    holding the step rows at [L, L + n_q)."""
    shape, out, lse, odt = _prepare(q, k_cache, v_cache, kv_lens, out_dtype, out, lse, return_lse)
    _check(k_step, "k_step", torch.bfloat16)
    _check(v_step, "v_step", torch.bfloat16)
    want = (shape.B, shape.n_q, shape.Hkv, shape.D)
    if tuple(k_step.shape) != want or tuple(v_step.shape) != want:
        raise ValueError(f"k_step and v_step must be [B, n_q, Hkv, D] = {want}")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    st_handle = _stream_handle(stream, q.device)
    if workspace is None:
        workspace = _cached_workspace(shape, 0, num_splits, q.device, st_handle)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ck_decode_attn_steps(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(kv_lens), _ptr(k_step), _ptr(v_step), ctypes.c_float(scale),
                                    _ptr(out), odt, _ptr(lse), _ptr(workspace), ws_bytes, num_splits,
                                    ctypes.c_void_p(st_handle))
    if st != 0:
        raise CkError(st, "ck_decode_attn_steps")
    return (out, lse) if (return_lse or lse is not None) else out


class PagedQ8Cache:
    """A paged INT8 KV cache in device memory: k/v codes int8 [num_pages, Hkv,
    page_tokens, D], k/v scales fp32 [num_pages, Hkv, page_tokens], and a
    block table int32 [B, max_pages] mapping each sequence's logical pages to
    pool pages (see ck_q8_cache).  Pages are the caller's to assign; lowering
    a sequence's kv_lens entry rolls it back."""

    def __init__(self, num_pages: int, page_tokens: int, Hkv: int, D: int, block_table: torch.Tensor,
                 device=None):
        device = device or block_table.device
        _check(block_table, "block_table", torch.int32)
        if block_table.dim() != 2:
            raise ValueError("block_table must be [B, max_pages]")
        self.k_codes = torch.zeros((num_pages, Hkv, page_tokens, D), dtype=torch.int8, device=device)
        self.v_codes = torch.zeros_like(self.k_codes)
        self.k_scales = torch.zeros((num_pages, Hkv, page_tokens), dtype=torch.float32, device=device)
        self.v_scales = torch.zeros_like(self.k_scales)
        self.block_table = block_table
        self.page_tokens, self.num_pages, self.Hkv, self.D = page_tokens, num_pages, Hkv, D

    @property
    def B(self) -> int:
        return self.block_table.shape[0]

    @property
    def max_pages(self) -> int:
        return self.block_table.shape[1]

    @property
    def capacity(self) -> int:
        return self.page_tokens * self.max_pages

    def c_struct(self) -> Q8CacheC:
        return Q8CacheC(self.k_codes.data_ptr(), self.v_codes.data_ptr(), self.k_scales.data_ptr(),
                        self.v_scales.data_ptr(), self.block_table.data_ptr(), self.page_tokens,
                        self.max_pages, self.num_pages)


def kv_append_q8(cache: PagedQ8Cache, k_new, v_new, start, stream=None):
    """Quantize k_new / v_new [B, n_new, Hkv, D] bf16 into the cache at
    positions start[b] + t (``ck_kv_append_q8``); start is int32 [B] on the
    device (usually kv_lens, which the caller then advances)."""
    _check(k_new, "k_new", torch.bfloat16)
    _check(v_new, "v_new", torch.bfloat16)
    if k_new.dim() != 4:
        raise ValueError("k_new must be [B, n_new, Hkv, D]")
    B, n_new, Hkv, D = k_new.shape
    _check_lens(start, B, "start")
    if tuple(v_new.shape) != tuple(k_new.shape) or (B, Hkv, D) != (cache.B, cache.Hkv, cache.D):
        raise ValueError("k_new / v_new must be [B, n_new, Hkv, D] matching the cache")
    shape = Shape(B, n_new, Hkv, Hkv, D, cache.capacity)
    cs = cache.c_struct()
    st_handle = _stream_handle(stream, k_new.device)
    st = lib().ck_kv_append_q8(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(start), ctypes.byref(cs),
                               ctypes.c_void_p(st_handle))
    if st != 0:
        raise CkError(st, "ck_kv_append_q8")


def decode_attn_q8(q, cache: PagedQ8Cache, kv_lens, *, scale: float | None = None, causal: bool = False,
                   out_dtype=torch.float32, out=None, lse=None, return_lse=False, workspace=None,
                   num_splits: int = 0, stream=None):
    """Decode attention over the paged INT8 cache (``ck_decode_attn_q8``)."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    _check(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, n_q, Hq, D]")
    B, n_q, Hq, D = q.shape
    if B != cache.B or D != cache.D:
        raise ValueError("q and the cache disagree on B or D")
    _check_lens(kv_lens, B)
    shape = Shape(B, n_q, Hq, cache.Hkv, D, cache.capacity)
    out, lse = _outputs(q, out_dtype, out, lse, return_lse)
    odt = CK_DT_BF16 if out_dtype == torch.bfloat16 else CK_DT_F32
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st_handle = _stream_handle(stream, q.device)
    if workspace is None:
        workspace = _cached_workspace(shape, 0, num_splits, q.device, st_handle)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cs = cache.c_struct()
    st = lib().ck_decode_attn_q8(ctypes.byref(shape), _ptr(q), ctypes.byref(cs), _ptr(kv_lens),
                                 ctypes.c_float(scale), 1 if causal else 0, _ptr(out), odt, _ptr(lse),
                                 _ptr(workspace), ws_bytes, num_splits, ctypes.c_void_p(st_handle))
    if st != 0:
        raise CkError(st, "ck_decode_attn_q8")
    return (out, lse) if (return_lse or lse is not None) else out
