"""CPU fp64 oracle for length-aware decode attention (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding)
never imports, links or calls it, and it imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain fp64 masked softmax attention
over the visible cells only; see that file's header for the definition and
the passages each step follows).  This module only builds it with gcc and
marshals arguments through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB, extra_flags: tuple = ()) -> str:
    """Compile ``oracle.c`` into a shared library with gcc and return its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", *extra_flags, src,
           "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str | None = None):
    """Load the compiled oracle (building it first if it is missing)."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        path = _LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    lib.ck_oracle_attn.restype = ctypes.c_int
    lib.ck_oracle_attn.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    lib.ck_oracle_attn_steps.restype = ctypes.c_int
    lib.ck_oracle_attn_steps.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.ck_oracle_attn_q8.restype = ci
    lib.ck_oracle_attn_q8.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_float, ci, ci, vp, vp, ci]
    lib.ck_oracle_q8_quantize_rows.restype = None
    lib.ck_oracle_q8_quantize_rows.argtypes = [ctypes.c_longlong, ci, vp, vp, vp]
    lib.ck_oracle_q8_append.restype = ci
    lib.ck_oracle_q8_append.argtypes = [ci, ci, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ck_oracle_topk.restype = ci
    lib.ck_oracle_topk.argtypes = [ci, ci, ci, ci, vp, vp, ci, ci, ci, vp]
    lib.ck_oracle_nthreads_default.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def _bits(a) -> np.ndarray:
    """bf16 data as a contiguous uint16 numpy array of its bit patterns."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            if a.dtype != torch.bfloat16:
                raise TypeError("oracle inputs must be bfloat16 tensors or uint16 bit arrays")
            return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy()
                                        .view(np.uint16))
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs must be bfloat16 tensors or uint16 bit arrays")
    return np.ascontiguousarray(a)


def _np(a, dtype) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def attn(q, k_cache, v_cache, kv_lens, scale: float, causal: bool = False, keep_mask=None,
         idx=None, idx_head_stride: int | None = None, num_splits: int = 0,
         nthreads: int = 0, lib=None):
    """Masked softmax attention in fp64 over the visible cells.

    q [B, n_q, Hq, D], k_cache / v_cache [B, cap, Hkv, D] (bf16 tensors or
    uint16 bit arrays), kv_lens [B] int32, keep_mask [B, n_q, Hkv, cap] uint8
    or None, idx [B, n_q, Hkv, W] or [B, n_q, W] int32 or None.
    Returns (out [B, n_q, Hq, D] float64, lse [B, n_q, Hq] float64).
    """
    lib = lib or load()
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    B, n_q, Hq, D = qb.shape
    Bk, cap, Hkv, Dk = kb.shape
    if vb.shape != kb.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k_cache and v_cache")
    lens = _np(kv_lens, np.int32).reshape(-1)
    if lens.shape[0] != B:
        raise ValueError("kv_lens must have B entries")
    mask_arr = None
    if keep_mask is not None:
        mask_arr = _np(keep_mask, np.uint8)
        if mask_arr.shape != (B, n_q, Hkv, cap):
            raise ValueError("keep_mask must be [B, n_q, Hkv, cap]")
    idx_arr, W, hs = None, 0, 0
    if idx is not None:
        idx_arr = _np(idx, np.int32)
        if idx_arr.ndim == 3:
            if idx_arr.shape[:2] != (B, n_q):
                raise ValueError("shared idx must be [B, n_q, W]")
            W, hs = idx_arr.shape[2], 0
        elif idx_arr.ndim == 4:
            if idx_arr.shape[:3] != (B, n_q, Hkv):
                raise ValueError("idx must be [B, n_q, Hkv, W]")
            W = idx_arr.shape[3]
            hs = W
        else:
            raise ValueError("idx must be 3-D or 4-D")
        if idx_head_stride is not None and idx_head_stride != hs:
            raise ValueError("idx_head_stride does not match idx's layout")
    out = np.empty((B, n_q, Hq, D), dtype=np.float64)
    lse = np.empty((B, n_q, Hq), dtype=np.float64)
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    st = lib.ck_oracle_attn(B, n_q, Hq, Hkv, D, cap, ptr(qb), ptr(kb), ptr(vb), ptr(lens),
                            ctypes.c_float(scale), 1 if causal else 0, ptr(mask_arr),
                            ptr(idx_arr), W, hs, num_splits, ptr(out), ptr(lse), _threads(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return out, lse


def attn_steps(q, k_cache, v_cache, kv_lens, k_step, v_step, scale: float, num_splits: int = 0,
               nthreads: int = 0, lib=None):
    """Attention of n_q verification queries over the cache prefix [0, L)
    plus their own step rows: query i sees step rows 0..i of
    k_step / v_step [B, n_q, Hkv, D] (not written into the cache).
    Returns (out [B, n_q, Hq, D] float64, lse [B, n_q, Hq] float64)."""
    lib = lib or load()
    qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
    ksb, vsb = _bits(k_step), _bits(v_step)
    B, n_q, Hq, D = qb.shape
    Bk, cap, Hkv, Dk = kb.shape
    if vb.shape != kb.shape or Bk != B or Dk != D:
        raise ValueError("shape mismatch between q, k_cache and v_cache")
    if ksb.shape != (B, n_q, Hkv, D) or vsb.shape != ksb.shape:
        raise ValueError("k_step / v_step must be [B, n_q, Hkv, D]")
    lens = _np(kv_lens, np.int32).reshape(-1)
    if lens.shape[0] != B:
        raise ValueError("kv_lens must have B entries")
    out = np.empty((B, n_q, Hq, D), dtype=np.float64)
    lse = np.empty((B, n_q, Hq), dtype=np.float64)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = lib.ck_oracle_attn_steps(B, n_q, Hq, Hkv, D, cap, ptr(qb), ptr(kb), ptr(vb), ptr(lens),
                                  ptr(ksb), ptr(vsb), ctypes.c_float(scale), num_splits, ptr(out),
                                  ptr(lse), _threads(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return out, lse


def q8_quantize(x, lib=None):
    """Rows of bf16 x [..., D] to (codes int8 [..., D], scales float32 [...])."""
    lib = lib or load()
    xb = _bits(x)
    D = xb.shape[-1]
    codes = np.empty(xb.shape, dtype=np.int8)
    scales = np.empty(xb.shape[:-1], dtype=np.float32)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    lib.ck_oracle_q8_quantize_rows(xb.size // D, D, ptr(xb), ptr(codes), ptr(scales))
    return codes, scales


def q8_append(k_new, v_new, start, block_table, kq, vq, ksc, vsc, lib=None):
    """Quantize k_new / v_new [B, n_new, Hkv, D] (bf16) into the paged cache
    (kq, vq int8 [num_pages, Hkv, page, D]; ksc, vsc float32 [num_pages,
    Hkv, page]; numpy arrays updated in place) at positions start[b] + t."""
    lib = lib or load()
    kb, vb = _bits(k_new), _bits(v_new)
    B, n_new, Hkv, D = kb.shape
    num_pages, page = kq.shape[0], kq.shape[2]
    bt = _np(block_table, np.int32)
    st = _np(start, np.int32).reshape(-1)
    for a, dt in ((kq, np.int8), (vq, np.int8), (ksc, np.float32), (vsc, np.float32)):
        if a.dtype != dt or not a.flags.c_contiguous:
            raise ValueError("paged cache arrays must be contiguous int8 / float32")
    if kq.shape != (num_pages, Hkv, page, D) or vq.shape != kq.shape or ksc.shape != kq.shape[:3] \
            or vsc.shape != ksc.shape or bt.shape[0] != B or st.shape[0] != B:
        raise ValueError("paged cache shape mismatch")
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    r = lib.ck_oracle_q8_append(B, n_new, Hkv, D, page, bt.shape[1], num_pages, ptr(kb), ptr(vb), ptr(st),
                                ptr(bt), ptr(kq), ptr(vq), ptr(ksc), ptr(vsc))
    if r != 0:
        raise RuntimeError(f"oracle failed with status {r}")


def topk(scores, kv_lens, k: int, tail: int = 0, causal: bool = False, lib=None) -> np.ndarray:
    """Top-k index lists: for each row of scores [B, n_q, Hs, cap] (float32),
    the min(k, n) best of the n cells before the window's last ``tail`` cells
    (larger score first, then smaller cell; NaN as -inf), ascending, then the
    tail cells, then -1.  Returns int32 [B, n_q, Hs, k + tail]."""
    lib = lib or load()
    sc = np.ascontiguousarray(np.asarray(scores, dtype=np.float32))
    if sc.ndim != 4:
        raise ValueError("scores must be [B, n_q, Hs, cap]")
    B, n_q, Hs, cap = sc.shape
    lens = _np(kv_lens, np.int32).reshape(-1)
    if lens.shape[0] != B:
        raise ValueError("kv_lens must have B entries")
    out = np.empty((B, n_q, Hs, k + tail), dtype=np.int32)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    r = lib.ck_oracle_topk(B, n_q, Hs, cap, ptr(sc), ptr(lens), int(k), int(tail), 1 if causal else 0, ptr(out))
    if r != 0:
        raise RuntimeError(f"oracle failed with status {r}")
    return out


def attn_q8(q, kq, vq, ksc, vsc, block_table, kv_lens, scale: float, causal: bool = False,
            num_splits: int = 0, nthreads: int = 0, lib=None):
    """Attention over the paged INT8 cache (kq/vq [num_pages, Hkv, page, D],
    ksc/vsc [num_pages, Hkv, page]; cell j of sequence b in page
    block_table[b, j // page], value code * scale).  q [B, n_q, Hq, D] bf16.
    Returns (out [B, n_q, Hq, D] float64, lse [B, n_q, Hq] float64)."""
    lib = lib or load()
    qb = _bits(q)
    B, n_q, Hq, D = qb.shape
    kq, vq = _np(kq, np.int8), _np(vq, np.int8)
    ksc, vsc = _np(ksc, np.float32), _np(vsc, np.float32)
    num_pages, Hkv, page, Dk = kq.shape
    bt = _np(block_table, np.int32)
    if Dk != D or vq.shape != kq.shape or ksc.shape != kq.shape[:3] or vsc.shape != ksc.shape:
        raise ValueError("paged cache shape mismatch")
    if bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    lens = _np(kv_lens, np.int32).reshape(-1)
    out = np.empty((B, n_q, Hq, D), dtype=np.float64)
    lse = np.empty((B, n_q, Hq), dtype=np.float64)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = lib.ck_oracle_attn_q8(B, n_q, Hq, Hkv, D, page, bt.shape[1], num_pages, ptr(qb), ptr(kq), ptr(vq),
                               ptr(ksc), ptr(vsc), ptr(bt), ptr(lens), ctypes.c_float(scale),
                               1 if causal else 0, num_splits, ptr(out), ptr(lse), _threads(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle failed with status {st}")
    return out, lse


def default_threads() -> int:
    """Worker threads for a call that asks for the default (nthreads <= 0):
    the host cores this process may run on, capped by OMP_NUM_THREADS when
    that is set (a shared host's CPU share)."""
    n = load().ck_oracle_nthreads_default()
    try:
        n = min(n, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        pass
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _threads(nthreads: int) -> int:
    return nthreads if nthreads > 0 else default_threads()
