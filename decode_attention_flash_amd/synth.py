"""Seeded synthetic inputs for decode attention.

This module only draws random tensors and index lists of the shapes and
value distributions of the decode workloads; it holds none of the attention
arithmetic.  Tests feed the same tensors to the HIP library and to the CPU
oracle, and the benchmark uses it to build its layer caches.

Value recipe: Q, K and V are N(0, 1) draws rounded to bf16.  Cache slots at
or beyond a sequence's filled length hold uniformly random 16-bit patterns
viewed as bf16 ("garbage"), which includes NaN and +-Inf encodings, unless
the caller asks for N(0, 1) there too.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def bf16_normal(shape, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """N(0, 1) draws rounded (RNE) to bfloat16."""
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def bf16_garbage(shape, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """Uniform random 16-bit patterns viewed as bfloat16 (NaN/Inf included)."""
    bits = torch.randint(-32768, 32768, shape, generator=gen, device=device, dtype=torch.int32)
    return bits.to(torch.int16).view(torch.bfloat16)


def kv_cache(B: int, cap: int, Hkv: int, D: int, fill_lens, seed: int, device="cpu",
             garbage: bool = True):
    """K and V caches [B, cap, Hkv, D] bf16.

    Slots j < fill_lens[b] hold N(0, 1) values drawn from a stream that does
    not depend on ``cap`` (so two caches of different capacity share the same
    filled prefix bit for bit); slots at or beyond it hold garbage (or more
    N(0, 1) values when ``garbage`` is False).
    """
    fill = [int(min(max(x, 0), cap)) for x in fill_lens]
    if len(fill) != B:
        raise ValueError("fill_lens must have B entries")
    gen = generator(seed, device)
    k = torch.empty((B, cap, Hkv, D), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    for b in range(B):
        n = fill[b]
        if n:
            k[b, :n] = bf16_normal((n, Hkv, D), gen, device)
            v[b, :n] = bf16_normal((n, Hkv, D), gen, device)
    tail_gen = generator(seed + 7919, device)
    for b in range(B):
        n = fill[b]
        if n < cap:
            if garbage:
                k[b, n:] = bf16_garbage((cap - n, Hkv, D), tail_gen, device)
                v[b, n:] = bf16_garbage((cap - n, Hkv, D), tail_gen, device)
            else:
                k[b, n:] = bf16_normal((cap - n, Hkv, D), tail_gen, device)
                v[b, n:] = bf16_normal((cap - n, Hkv, D), tail_gen, device)
    return k, v


def queries(B: int, n_q: int, Hq: int, D: int, seed: int, device="cpu") -> torch.Tensor:
    return bf16_normal((B, n_q, Hq, D), generator(seed + 104729, device), device)


def ragged_lens(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Per-sequence lengths drawn uniformly from the inclusive range [lo, hi]."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)


def topk_lists(B: int, n_q: int, Hkv: int, n_kv: int, n_sel: int, tail: int, seed: int):
    """Index lists [B, n_q, Hkv, n_sel + tail] int32.

    Each list holds ``n_sel`` distinct sorted random cells from
    [0, n_kv - tail) followed by the last ``tail`` cells [n_kv - tail, n_kv).
    """
    if n_sel > n_kv - tail:
        raise ValueError("not enough cells to select from")
    rng = np.random.default_rng(seed)
    W = n_sel + tail
    out = np.empty((B, n_q, Hkv, W), dtype=np.int32)
    tail_cells = np.arange(n_kv - tail, n_kv, dtype=np.int32)
    for b in range(B):
        for i in range(n_q):
            for g in range(Hkv):
                sel = rng.choice(n_kv - tail, size=n_sel, replace=False)
                out[b, i, g, :n_sel] = np.sort(sel).astype(np.int32)
                out[b, i, g, n_sel:] = tail_cells
    return out


def index_scores(B: int, n_q: int, Hs: int, cap: int, seed: int, device="cpu") -> torch.Tensor:
    """Selection scores [B, n_q, Hs, cap] float32 ~ N(0, 1): one score per
    cache cell for each query and score head (the indexer's output, which
    needs trained weights, stands in as noise)."""
    g = generator(seed, device)
    return torch.randn((B, n_q, Hs, cap), generator=g, device=device, dtype=torch.float32)


def block_lists(B: int, n_q: int, Hkv: int, n_kv: int, n_blocks: int, block: int, tail: int,
                seed: int) -> np.ndarray:
    """Index lists [B, n_q, Hkv, n_blocks * block + tail] int32 whose cells
    come in runs: ``n_blocks`` distinct random aligned blocks of ``block``
    cells from [0, n_kv - tail), in increasing order, followed by the last
    ``tail`` cells.  A selection made over pooled block keys looks like this:
    the same number of cells as a scattered selection, in few places."""
    n_avail = (n_kv - tail) // block
    if n_blocks > n_avail:
        raise ValueError("not enough blocks to select from")
    rng = np.random.default_rng(seed)
    out = np.empty((B, n_q, Hkv, n_blocks * block + tail), dtype=np.int32)
    tail_cells = np.arange(n_kv - tail, n_kv, dtype=np.int32)
    offs = np.arange(block, dtype=np.int64)
    for b in range(B):
        for i in range(n_q):
            for g in range(Hkv):
                blocks = np.sort(rng.choice(n_avail, size=n_blocks, replace=False))
                cells = (blocks.reshape(-1, 1) * block + offs.reshape(1, -1)).reshape(-1)
                out[b, i, g, : n_blocks * block] = cells.astype(np.int32)
                out[b, i, g, n_blocks * block:] = tail_cells
    return out


def mask_from_lists(idx: np.ndarray, cap: int) -> np.ndarray:
    """keep_mask [B, n_q, Hkv, cap] uint8 with 1 exactly at the listed cells
    that fall in [0, cap)."""
    B, n_q, Hkv, W = idx.shape
    m = np.zeros((B, n_q, Hkv, cap), dtype=np.uint8)
    for b in range(B):
        for i in range(n_q):
            for g in range(Hkv):
                cells = idx[b, i, g]
                cells = cells[(cells >= 0) & (cells < cap)]
                m[b, i, g, cells] = 1
    return m


def counting_values(cap: int, Hkv: int, D: int, nbits: int) -> torch.Tensor:
    """V [1, cap, Hkv, D] bf16 with V[j, d] = bit d of j for d < nbits,
    V[j, nbits] = 1 and 0 elsewhere (exact in bf16)."""
    if nbits + 1 > D:
        raise ValueError("D too small for the counting construction")
    j = torch.arange(cap, dtype=torch.int64).view(cap, 1)
    d = torch.arange(nbits, dtype=torch.int64).view(1, nbits)
    bits = ((j >> d) & 1).to(torch.float32)
    v = torch.zeros((1, cap, Hkv, D), dtype=torch.float32)
    v[0, :, :, :nbits] = bits.view(cap, 1, nbits)
    v[0, :, :, nbits] = 1.0
    return v.to(torch.bfloat16)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
