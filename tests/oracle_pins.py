"""Independent checks that pin the CPU oracle (shared by the oracle tests and
the mutation test, which runs them against deliberately broken copies).

Nothing here re-types the oracle's formula.  Each check compares it with
something fixed from outside it:
  * torch's scaled_dot_product_attention and logsumexp in float64 (a library
    routine) with an explicit boolean mask, K/V expanded over the GQA group,
    at head dims 4, 16, 128 and 256;
  * attention written out in plain Python floats with math.exp, on tiny
    shapes (an implementation independent of both the oracle and torch);
  * closed forms (uniform V, one visible key, K = 0, two keys);
  * invariants (split count, gather vs mask, causal row vs a shorter plain
    decode, head permutation within a group, duplicate cells);
  * for the step-row merge: SDPA over a cache that holds the step rows after
    the prefix, with the bottom-right causal mask, and its closed forms;
  * for the paged INT8 cache: the quantizer's error bound, extremes and an
    exact round trip; SDPA over the pages gathered through the block table;
    page-pool permutation; append placement and rollback.
Every check returns the largest deviation it saw, so a caller can assert a
bound or, for a planted mistake, that some bound is broken.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from decode_attention_flash_amd import synth

TOL = 1e-12


def f64(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.float64)


def sdpa_reference(q, k, v, kv_lens, scale, causal, keep_mask=None, idx=None, bias=None):
    """Attention by torch SDPA (float64, CPU) with an explicit boolean mask.

    Returns (out [B, n_q, Hq, D], lse [B, n_q, Hq]) with fully masked rows set
    to 0 / -inf (SDPA itself yields NaN there).  ``idx`` lists must hold
    distinct cells, since a boolean mask can express a set only; ``bias`` is
    an optional float tensor [B, n_q, Hq, cap] added to visible scores.
    """
    B, n_q, Hq, D = q.shape
    _, cap, Hkv, _ = k.shape
    G = Hq // Hkv
    qd = f64(q).permute(0, 2, 1, 3)                                    # B,Hq,n_q,D
    kd = f64(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)        # B,Hq,cap,D
    vd = f64(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    lens = torch.as_tensor(np.asarray(kv_lens), dtype=torch.int64).clamp(0, cap)
    j = torch.arange(cap).view(1, 1, cap)
    i = torch.arange(n_q).view(1, n_q, 1)
    L = lens.view(B, 1, 1)
    lim = (L - n_q + i + 1).clamp(min=0) if causal else L.expand(B, n_q, 1)
    lim = torch.minimum(lim, L)
    vis = (j < lim)                                                    # B,n_q,cap
    # cells at or past L may hold garbage (NaN/Inf): give the library zeros
    # there, since a masked weight of 0 times NaN would still be NaN
    filled = (torch.arange(cap).view(1, 1, cap, 1) < lens.view(B, 1, 1, 1))
    kd = torch.where(filled, kd, torch.zeros_like(kd))
    vd = torch.where(filled, vd, torch.zeros_like(vd))
    vis = vis.view(B, 1, n_q, cap).expand(B, Hq, n_q, cap).clone()
    if keep_mask is not None:
        km = torch.as_tensor(np.asarray(keep_mask)).bool()           # B,n_q,Hkv,cap
        km = km.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
        vis &= km
    if idx is not None:
        idx = np.asarray(idx)
        sel = torch.zeros((B, Hq, n_q, cap), dtype=torch.bool)
        for b in range(B):
            for ii in range(n_q):
                for h in range(Hq):
                    lst = idx[b, ii] if idx.ndim == 3 else idx[b, ii, h // G]
                    lst = lst[(lst >= 0) & (lst < cap)]
                    sel[b, h, ii, torch.as_tensor(lst, dtype=torch.int64)] = True
        vis &= sel
    mask = vis
    if bias is not None:
        fb = f64(torch.as_tensor(bias)).permute(0, 2, 1, 3)
        mask = torch.where(vis, fb, torch.full_like(fb, -math.inf))
    out = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask,
                                                         scale=float(scale))
    scores = torch.matmul(qd, kd.transpose(-1, -2).contiguous()) * float(scale)
    if bias is not None:
        scores = scores + torch.where(vis, fb, torch.zeros_like(fb))
    scores = scores.masked_fill(~vis, -math.inf)
    lse = torch.logsumexp(scores, dim=-1)
    empty = ~vis.any(dim=-1)
    out = torch.where(empty.unsqueeze(-1), torch.zeros_like(out), out)
    lse = torch.where(empty, torch.full_like(lse, -math.inf), lse)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


def max_dev(a, b) -> float:
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    both_ninf = np.isneginf(a) & np.isneginf(b)
    if np.any(np.isnan(a)) or np.any(np.isnan(b)):
        return math.inf
    with np.errstate(invalid="ignore"):
        d = np.where(both_ninf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0


def small_case(B=2, n_q=3, Hq=4, Hkv=2, D=16, cap=40, lens=(37, 5), seed=0, garbage=True):
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, seed, garbage=garbage)
    q = synth.queries(B, n_q, Hq, D, seed)
    return q, k, v, np.asarray(lens, dtype=np.int32)


# ---------------------------------------------------------------- checks ----

def check_sdpa_dense(lib) -> float:
    worst = 0.0
    for causal in (False, True):
        for D in (4, 16):
            q, k, v, lens = small_case(D=D, lens=(37, 2), seed=D + causal)
            scale = 1.0 / math.sqrt(D)
            o, l = oracle.attn(q, k, v, lens, scale, causal, lib=lib)
            ro, rl = sdpa_reference(q, k, v, lens, np.float32(scale), causal)
            worst = max(worst, max_dev(o, ro), max_dev(l, rl))
    return worst


def check_sdpa_wide_heads(lib) -> float:
    """SDPA at the head dims the kernels serve (128 and 256): dense, causal,
    keep_mask and gather sets, B = 2, cap = 64."""
    worst = 0.0
    rng = np.random.default_rng(17)
    for D in (128, 256):
        q, k, v, lens = small_case(B=2, n_q=3, Hq=4, Hkv=2, D=D, cap=64, lens=(61, 3), seed=D)
        scale = np.float32(1.0 / math.sqrt(D))
        km = (rng.random((2, 3, 2, 64)) < 0.6).astype(np.uint8)
        idx = gather_lists(2, 3, 2, 64, 20, seed=D + 1)
        for causal in (False, True):
            for kw in ({}, {"keep_mask": km}, {"idx": idx}):
                o, l = oracle.attn(q, k, v, lens, float(scale), causal, lib=lib, **kw)
                ro, rl = sdpa_reference(q, k, v, lens, scale, causal, **kw)
                worst = max(worst, max_dev(o, ro), max_dev(l, rl))
    return worst


def attn_brute(q, k, v, lens, scale, causal, keep_mask=None, idx=None):
    """Attention written out with Python floats and math.exp, cell by cell:
    for each (b, i, h) the visible cells in order, their scores, the max, the
    exponentials, their sum, the weighted V rows and the log-sum-exp.  Small
    shapes only."""
    B, n_q, Hq, D = q.shape
    cap, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    Q, K, V = q.float().tolist(), k.float().tolist(), v.float().tolist()
    sc = float(np.float32(scale))
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(n_q)] for _ in range(B)]
    lse = [[[-math.inf] * Hq for _ in range(n_q)] for _ in range(B)]
    for b in range(B):
        L = min(max(int(lens[b]), 0), cap)
        for i in range(n_q):
            lim = min(max(L - n_q + i + 1, 0), L) if causal else L
            for h in range(Hq):
                g = h // G
                if idx is None:
                    cells = [j for j in range(lim) if keep_mask is None or keep_mask[b][i][g][j]]
                else:
                    lst = idx[b][i] if np.asarray(idx).ndim == 3 else idx[b][i][g]
                    cells = [int(j) for j in lst if 0 <= int(j) < lim]
                if not cells:
                    continue
                s = [sc * sum(Q[b][i][h][d] * K[b][j][g][d] for d in range(D)) for j in cells]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                den = math.fsum(e)
                for d in range(D):
                    out[b][i][h][d] = math.fsum(w * V[b][j][g][d] for w, j in zip(e, cells)) / den
                lse[b][i][h] = m + math.log(den)
    return np.array(out), np.array(lse)


def check_python_bruteforce(lib) -> float:
    """Against attention written out in plain Python (math.exp) on tiny
    shapes (D = 4, cap = 8, two query heads on one KV head, n_q <= 3):
    dense, causal, keep_mask and gather sets, with garbage past the length
    and empty rows."""
    worst = 0.0
    rng = np.random.default_rng(19)
    for n_q in (1, 2, 3):
        for lens in ((8, 0), (5, 2), (3, 8)):
            q, k, v, L = small_case(B=2, n_q=n_q, Hq=2, Hkv=1, D=4, cap=8, lens=lens, seed=10 * n_q + lens[1])
            km = (rng.random((2, n_q, 1, 8)) < 0.5).astype(np.uint8)
            idx = rng.integers(-2, 10, size=(2, n_q, 1, 6)).astype(np.int32)
            for causal in (False, True):
                for kw in ({}, {"keep_mask": km}, {"idx": idx}):
                    o, l = oracle.attn(q, k, v, L, 0.7, causal, lib=lib, **kw)
                    ro, rl = attn_brute(q, k, v, L, 0.7, causal, **kw)
                    worst = max(worst, max_dev(o, ro), max_dev(l, rl))
    return worst


def check_sdpa_mask(lib) -> float:
    q, k, v, lens = small_case(seed=3)
    rng = np.random.default_rng(3)
    km = (rng.random((2, 3, 2, 40)) < 0.5).astype(np.uint8)
    worst = 0.0
    for causal in (False, True):
        o, l = oracle.attn(q, k, v, lens, 0.25, causal, keep_mask=km, lib=lib)
        ro, rl = sdpa_reference(q, k, v, lens, np.float32(0.25), causal, keep_mask=km)
        worst = max(worst, max_dev(o, ro), max_dev(l, rl))
    return worst


def gather_lists(B, n_q, Hkv, cap, W, seed, shared=False):
    """Distinct cells per list, including out-of-range entries (-3, cap + 2)
    and the boundary cells 0, L-1 and L of a causal limit."""
    rng = np.random.default_rng(seed)
    shape = (B, n_q, W) if shared else (B, n_q, Hkv, W)
    out = np.empty(shape, dtype=np.int32)
    for pos in np.ndindex(*shape[:-1]):
        cells = rng.choice(cap, size=W - 2, replace=False).astype(np.int32)
        out[pos] = np.concatenate([cells, np.array([-3, cap + 2], dtype=np.int32)])
        rng.shuffle(out[pos])
    return out


def check_sdpa_gather(lib) -> float:
    q, k, v, lens = small_case(seed=5)
    worst = 0.0
    for shared in (False, True):
        for causal in (False, True):
            idx = gather_lists(2, 3, 2, 40, 12, seed=7 + shared, shared=shared)
            o, l = oracle.attn(q, k, v, lens, 0.3, causal, idx=idx, lib=lib)
            ro, rl = sdpa_reference(q, k, v, lens, np.float32(0.3), causal, idx=idx)
            worst = max(worst, max_dev(o, ro), max_dev(l, rl))
    # a list that names every cell up to and including the causal limit of
    # each query: the entry at the limit itself must be dropped
    B, n_q, cap = 1, 3, 40
    q1, k1, v1, _ = small_case(B=1, lens=(20,), seed=11)
    lens1 = np.array([20], dtype=np.int32)
    idx = np.tile(np.arange(0, 24, dtype=np.int32), (1, n_q, 2, 1))
    o, l = oracle.attn(q1, k1, v1, lens1, 0.3, True, idx=idx, lib=lib)
    ro, rl = sdpa_reference(q1, k1, v1, lens1, np.float32(0.3), True, idx=idx)
    return max(worst, max_dev(o, ro), max_dev(l, rl))


def check_duplicates(lib) -> float:
    """A cell listed twice weighs twice: the same as adding ln 2 to its score."""
    q, k, v, lens = small_case(B=1, lens=(30,), seed=13)
    lens = np.array([30], dtype=np.int32)
    base = np.array([1, 4, 9, 16, 25, 29], dtype=np.int32)
    lst = np.concatenate([base, base[[2]]])
    idx = np.tile(lst, (1, 3, 2, 1))
    o, l = oracle.attn(q, k, v, lens, 0.3, False, idx=idx, lib=lib)
    bias = np.zeros((1, 3, 4, 40))
    bias[..., 9] = math.log(2.0)
    ro, rl = sdpa_reference(q, k, v, lens, np.float32(0.3), False,
                            idx=np.tile(base, (1, 3, 2, 1)), bias=bias)
    return max(max_dev(o, ro), max_dev(l, rl))


def check_closed_forms(lib) -> float:
    worst = 0.0
    B, n_q, Hq, Hkv, D, cap = 1, 2, 4, 2, 8, 16
    q = synth.queries(B, n_q, Hq, D, 21)
    k, _ = synth.kv_cache(B, cap, Hkv, D, [12], 21)
    lens = np.array([12], dtype=np.int32)
    # uniform V: every visible row equals the same vector -> output is that vector
    row = synth.bf16_normal((Hkv, D), synth.generator(5))
    v = row.view(1, 1, Hkv, D).expand(B, cap, Hkv, D).contiguous()
    o, _ = oracle.attn(q, k, v, lens, 0.5, True, lib=lib)
    expect = f64(row).repeat_interleave(Hq // Hkv, dim=0).numpy()
    worst = max(worst, max_dev(o[0, 0], expect), max_dev(o[0, 1], expect))
    # one visible key: output is exactly its V row, lse is exactly its score
    k2, v2 = synth.kv_cache(B, cap, Hkv, D, [1], 22)
    o, l = oracle.attn(q, k2, v2, np.array([1], np.int32), 0.5, False, lib=lib)
    for h in range(Hq):
        worst = max(worst, max_dev(o[0, 0, h], f64(v2[0, 0, h // 2]).numpy()))
        sc = 0.5 * float(np.dot(f64(q[0, 0, h]).numpy(), f64(k2[0, 0, h // 2]).numpy()))
        worst = max(worst, abs(l[0, 0, h] - sc))
    # K = 0: uniform weights -> mean of the visible V rows, lse = ln(n)
    kz = torch.zeros_like(k)
    _, v3 = synth.kv_cache(B, cap, Hkv, D, [12], 23)
    o, l = oracle.attn(q, kz, v3, lens, 0.5, False, lib=lib)
    mean = f64(v3[0, :12]).mean(dim=0).repeat_interleave(2, dim=0).numpy()
    worst = max(worst, max_dev(o[0, 0], mean), float(np.max(np.abs(l - math.log(12)))))
    # two keys with score gap delta: o = sigma(delta) v1 + (1 - sigma(delta)) v2
    o, l = oracle.attn(q, k, v3, np.array([2], np.int32), 0.5, False, lib=lib)
    for h in range(Hq):
        qh = f64(q[0, 0, h]).numpy()
        s1 = 0.5 * float(np.dot(qh, f64(k[0, 0, h // 2]).numpy()))
        s2 = 0.5 * float(np.dot(qh, f64(k[0, 1, h // 2]).numpy()))
        sig = 1.0 / (1.0 + math.exp(-(s1 - s2)))
        exp_o = sig * f64(v3[0, 0, h // 2]).numpy() + (1 - sig) * f64(v3[0, 1, h // 2]).numpy()
        worst = max(worst, max_dev(o[0, 0, h], exp_o))
        lse2 = max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2)))
        worst = max(worst, abs(l[0, 0, h] - lse2))
    return worst


def check_split_invariance(lib) -> float:
    q, k, v, lens = small_case(D=16, lens=(37, 29), seed=31)
    ref, rl = oracle.attn(q, k, v, lens, 0.25, True, lib=lib)
    worst = 0.0
    for S in (1, 2, 7, 64):
        o, l = oracle.attn(q, k, v, lens, 0.25, True, num_splits=S, lib=lib)
        worst = max(worst, max_dev(o, ref), max_dev(l, rl))
    return worst


def check_causal_rows(lib) -> float:
    """Causal row i equals a plain single-query decode of length L - n_q + i + 1."""
    q, k, v, lens = small_case(D=16, lens=(37, 5), seed=41)
    n_q = q.shape[1]
    o, l = oracle.attn(q, k, v, lens, 0.25, True, lib=lib)
    worst = 0.0
    for i in range(n_q):
        li = np.maximum(lens - n_q + i + 1, 0).astype(np.int32)
        oi, lsi = oracle.attn(q[:, i:i + 1].contiguous(), k, v, li, 0.25, False, lib=lib)
        worst = max(worst, max_dev(o[:, i], oi[:, 0]), max_dev(l[:, i], lsi[:, 0]))
    return worst


def check_head_permutation(lib) -> float:
    q, k, v, lens = small_case(Hq=6, Hkv=2, D=8, seed=51)
    o, _ = oracle.attn(q, k, v, lens, 0.3, False, lib=lib)
    perm = torch.tensor([2, 0, 1, 4, 5, 3])            # permutes within each group of 3
    op, _ = oracle.attn(q[:, :, perm].contiguous(), k, v, lens, 0.3, False, lib=lib)
    return max_dev(op, o[:, :, perm.numpy()])


def steps_case(B=2, n_q=3, Hq=4, Hkv=2, D=16, cap=48, lens=(37, 0), seed=61):
    """A cache with garbage past the prefix, and separate step rows."""
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, seed)
    q = synth.queries(B, n_q, Hq, D, seed)
    gen = synth.generator(seed + 1)
    ks = synth.bf16_normal((B, n_q, Hkv, D), gen)
    vs = synth.bf16_normal((B, n_q, Hkv, D), gen)
    return q, k, v, np.asarray(lens, dtype=np.int32), ks, vs


def check_sdpa_steps(lib) -> float:
    """Step rows merged into the prefix equal SDPA over a cache holding the
    step rows at [L, L + n_q) under the bottom-right causal mask."""
    worst = 0.0
    for n_q, lens in ((3, (37, 0)), (1, (12, 1)), (5, (20, 43))):
        q, k, v, L, ks, vs = steps_case(n_q=n_q, lens=lens, seed=60 + n_q)
        o, l = oracle.attn_steps(q, k, v, L, ks, vs, 0.3, lib=lib)
        kc, vc = k.clone(), v.clone()
        for b in range(q.shape[0]):
            kc[b, L[b]:L[b] + n_q] = ks[b]
            vc[b, L[b]:L[b] + n_q] = vs[b]
        ro, rl = sdpa_reference(q, kc, vc, L + n_q, np.float32(0.3), True)
        worst = max(worst, max_dev(o, ro), max_dev(l, rl))
    return worst


def check_steps_closed_forms(lib) -> float:
    """Empty prefix: the first query sees only its own step row (output = that
    V row, lse = its score); with K = 0 query i averages step rows 0..i."""
    worst = 0.0
    q, k, v, L, ks, vs = steps_case(B=1, n_q=3, lens=(0,), seed=71)
    o, l = oracle.attn_steps(q, k, v, L, ks, vs, 0.3, lib=lib)
    for h in range(4):
        worst = max(worst, max_dev(o[0, 0, h], f64(vs[0, 0, h // 2]).numpy()))
        sc = float(np.float32(0.3)) * float(np.dot(f64(q[0, 0, h]).numpy(), f64(ks[0, 0, h // 2]).numpy()))
        worst = max(worst, abs(l[0, 0, h] - sc))
    o, _ = oracle.attn_steps(q, k, v, L, torch.zeros_like(ks), vs, 0.3, lib=lib)
    for i in range(3):
        mean = f64(vs[0, :i + 1]).mean(dim=0).repeat_interleave(2, dim=0).numpy()
        worst = max(worst, max_dev(o[0, i], mean))
    return worst


# ------------------------------------------------------- paged INT8 cache ----

def check_q8_quantize(lib) -> float:
    """Codes in [-127, 127]; the largest |x| maps to +-127; |x - code*scale| is
    at most half a step; negation is symmetric; zero rows give scale 0; rows
    k * 2^e (integers |k| <= 127, one of them 127) round-trip exactly."""
    worst = 0.0
    x = synth.bf16_normal((48, 64), synth.generator(81)) * 3
    x[5] = 0
    codes, sc = oracle.q8_quantize(x, lib=lib)
    xd = f64(x).numpy()
    worst = max(worst, float(np.max(np.abs(codes.astype(np.int64))) > 127))
    for r in range(x.shape[0]):
        if sc[r] == 0:
            worst = max(worst, float(np.any(codes[r] != 0)), float(np.any(xd[r] != 0)))
            continue
        err = np.abs(xd[r] - codes[r].astype(np.float64) * float(sc[r]))
        worst = max(worst, float(np.max(np.maximum(err - 0.5 * float(sc[r]) * (1 + 1e-5), 0))))
        worst = max(worst, float(abs(int(codes[r][np.argmax(np.abs(xd[r]))])) != 127))
    cn, sn = oracle.q8_quantize(-x, lib=lib)
    worst = max(worst, float(np.any(cn != -codes)), float(np.any(sn != sc)))
    gen = np.random.default_rng(82)
    k = gen.integers(-127, 128, size=(8, 32))
    k[:, 3] = 127 * np.where(gen.random(8) < 0.5, 1, -1)
    e = gen.integers(-20, 20, size=(8, 1))
    xr = torch.from_numpy(k * np.exp2(e.astype(np.float64))).to(torch.bfloat16)
    cr, sr = oracle.q8_quantize(xr, lib=lib)
    worst = max(worst, float(np.any(cr != k)), float(np.max(np.abs(sr - np.exp2(e[:, 0])))))
    return worst


def q8_case(B=2, n_q=3, Hq=4, Hkv=2, D=16, page=8, max_pages=4, num_pages=9, seed=91):
    gen = np.random.default_rng(seed)
    kq = gen.integers(-127, 128, size=(num_pages, Hkv, page, D)).astype(np.int8)
    vq = gen.integers(-127, 128, size=(num_pages, Hkv, page, D)).astype(np.int8)
    ksc = (gen.random((num_pages, Hkv, page)) * 0.05 + 0.001).astype(np.float32)
    vsc = (gen.random((num_pages, Hkv, page)) * 0.05 + 0.001).astype(np.float32)
    bt = np.stack([gen.permutation(num_pages)[:max_pages] for _ in range(B)]).astype(np.int32)
    q = synth.queries(B, n_q, Hq, D, seed)
    return q, kq, vq, ksc, vsc, bt


def q8_dense(codes, scales, bt, num_pages):
    """[B, max_pages * page, Hkv, D] float64 view of the pages ([num_pages,
    Hkv, page, D]) through the block table (invalid page ids give zeros)."""
    B, max_pages = bt.shape
    page = codes.shape[2]
    vals = (codes.astype(np.float64) * scales.astype(np.float64)[..., None]).transpose(0, 2, 1, 3)
    out = np.zeros((B, max_pages * page, codes.shape[1], codes.shape[3]), dtype=np.float64)
    for b in range(B):
        for lp in range(max_pages):
            pg = bt[b, lp]
            if 0 <= pg < num_pages:
                out[b, lp * page:(lp + 1) * page] = vals[pg]
    return torch.from_numpy(out)


def check_q8_sdpa(lib) -> float:
    """Attention over the paged INT8 cache equals SDPA over the dequantized
    pages gathered through the block table (dense and causal, a page id
    outside the pool reading as zeros)."""
    worst = 0.0
    q, kq, vq, ksc, vsc, bt = q8_case()
    bt[1, 1] = 40   # outside the pool of 9 pages: its cells read as zeros
    for causal in (False, True):
        lens = np.array([29, 17], dtype=np.int32)
        o, l = oracle.attn_q8(q, kq, vq, ksc, vsc, bt, lens, 0.3, causal, lib=lib)
        kd, vd = q8_dense(kq, ksc, bt, 9), q8_dense(vq, vsc, bt, 9)
        ro, rl = sdpa_reference(q, kd, vd, lens, np.float32(0.3), causal)
        worst = max(worst, max_dev(o, ro), max_dev(l, rl))
    return worst


def check_q8_page_permutation(lib) -> float:
    """Moving pages around the pool (and the block table with them) leaves the
    result bit-identical."""
    q, kq, vq, ksc, vsc, bt = q8_case(seed=92)
    lens = np.array([31, 9], dtype=np.int32)
    o, l = oracle.attn_q8(q, kq, vq, ksc, vsc, bt, lens, 0.25, True, lib=lib)
    perm = np.random.default_rng(93).permutation(9)      # new slot of old page p: perm[p]
    inv = np.argsort(perm)
    o2, l2 = oracle.attn_q8(q, kq[inv], vq[inv], ksc[inv], vsc[inv], perm[bt].astype(np.int32), lens,
                            0.25, True, lib=lib)
    return float(not (np.array_equal(o, o2) and np.array_equal(l, l2)))


def check_q8_append(lib) -> float:
    """Appended rows land at block_table[b][pos // page], row pos % page, as
    the quantizer's codes; a rollback (lower start) overwrites from there and
    leaves the rows past the new end as they were."""
    B, Hkv, D, page, max_pages, num_pages = 2, 2, 16, 8, 4, 9
    gen = np.random.default_rng(94)
    bt = np.stack([gen.permutation(num_pages)[:max_pages] for _ in range(B)]).astype(np.int32)
    kq = np.zeros((num_pages, Hkv, page, D), np.int8)
    vq = np.zeros_like(kq)
    ksc = np.zeros((num_pages, Hkv, page), np.float32)
    vsc = np.zeros_like(ksc)
    g0 = synth.generator(95)
    a_k, a_v = synth.bf16_normal((B, 6, Hkv, D), g0), synth.bf16_normal((B, 6, Hkv, D), g0)
    b_k, b_v = synth.bf16_normal((B, 2, Hkv, D), g0), synth.bf16_normal((B, 2, Hkv, D), g0)
    start = np.array([5, 27], dtype=np.int32)           # the second runs past capacity 32
    oracle.q8_append(a_k, a_v, start, bt, kq, vq, ksc, vsc, lib=lib)
    oracle.q8_append(b_k, b_v, start + 2, bt, kq, vq, ksc, vsc, lib=lib)   # rolled back to +2
    worst = 0.0
    for b in range(B):
        for t, (src_k, src_v) in enumerate([(a_k[b, 0], a_v[b, 0]), (a_k[b, 1], a_v[b, 1]),
                                            (b_k[b, 0], b_v[b, 0]), (b_k[b, 1], b_v[b, 1]),
                                            (a_k[b, 4], a_v[b, 4]), (a_k[b, 5], a_v[b, 5])]):
            pos = int(start[b]) + t
            if pos >= page * max_pages:
                continue
            pg, r = bt[b, pos // page], pos % page
            ck, sk = oracle.q8_quantize(src_k, lib=lib)
            cv, sv = oracle.q8_quantize(src_v, lib=lib)
            worst = max(worst, float(np.any(kq[pg, :, r] != ck)), float(np.any(ksc[pg, :, r] != sk)),
                        float(np.any(vq[pg, :, r] != cv)), float(np.any(vsc[pg, :, r] != sv)))
    untouched = np.ones(num_pages, bool)
    untouched[bt.reshape(-1)] = False
    worst = max(worst, float(np.any(kq[untouched] != 0)))
    return worst


# ---------------------------------------------------------------- top-k ----

def topk_brute(scores, lens, k, tail, causal):
    """Pure-Python top-k lists: a candidate is selected when fewer than k
    candidates beat it (a larger score, or the same score at a smaller cell;
    NaN counts as -inf)."""
    B, n_q, Hs, cap = scores.shape
    out = np.full((B, n_q, Hs, k + tail), -1, dtype=np.int64)
    for b in range(B):
        L = min(max(int(lens[b]), 0), cap)
        for i in range(n_q):
            lim = min(max(L - n_q + i + 1, 0), L) if causal else L
            n = max(0, lim - tail)
            for h in range(Hs):
                v = [float(x) for x in scores[b, i, h, :n]]
                v = [-math.inf if math.isnan(x) else x for x in v]
                chosen = []
                for c in range(n):
                    beaten = sum(1 for d in range(n) if v[d] > v[c] or (v[d] == v[c] and d < c))
                    if beaten < k:
                        chosen.append(c)
                row = chosen + list(range(n, lim))
                out[b, i, h, :len(row)] = row
    return out


def check_topk_brute_force(lib) -> float:
    """Against the brute force on small rows with many ties (small integer
    scores), NaN, -inf / +inf and signed zeros, causal windows, two score
    heads, lengths past the capacity and k larger than the candidates."""
    bad = 0
    gen = np.random.default_rng(101)
    for trial in range(40):
        B, n_q, Hs, cap = int(gen.integers(1, 3)), int(gen.integers(1, 4)), int(gen.integers(1, 3)), \
            int(gen.integers(1, 40))
        sc = gen.integers(-3, 4, size=(B, n_q, Hs, cap)).astype(np.float32)
        specials = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0], dtype=np.float32)
        pick = gen.random(sc.shape) < 0.15
        sc[pick] = specials[gen.integers(0, len(specials), size=int(pick.sum()))]
        lens = gen.integers(-2, cap + 3, size=B).astype(np.int32)
        k, tail, causal = int(gen.integers(1, 12)), int(gen.integers(0, 5)), bool(trial % 2)
        got = oracle.topk(sc, lens, k, tail, causal, lib=lib)
        bad += int(not np.array_equal(got, topk_brute(sc, lens, k, tail, causal)))
    return float(bad)


def check_topk_closed_forms(lib) -> float:
    """Scores rising with the cell select the last k candidates, falling
    scores the first k, equal scores the first k (lowest cell first); with
    k >= n every candidate; an empty window gives -1 throughout."""
    bad = 0
    cap, k, tail = 50, 7, 3
    lens = np.array([50, 31, 2, 0], dtype=np.int32)
    cells = np.arange(cap, dtype=np.float32)
    for kind in ("rise", "fall", "flat"):
        v = {"rise": cells, "fall": -cells, "flat": np.full(cap, 0.5, np.float32)}[kind]
        sc = np.broadcast_to(v, (4, 1, 1, cap)).copy()
        got = oracle.topk(sc, lens, k, tail, lib=lib)
        for b, L in enumerate(lens):
            n = max(0, int(L) - tail)
            m = min(k, n)
            sel = list(range(n - m, n)) if kind == "rise" else list(range(m))
            want = sel + list(range(n, int(L)))
            want += [-1] * (k + tail - len(want))
            bad += int(list(got[b, 0, 0]) != want)
    return float(bad)


def check_topk_permutation(lib) -> float:
    """Distinct scores moved between cells by a permutation: the selected
    cells move with them."""
    gen = np.random.default_rng(103)
    cap, k, tail = 300, 40, 5
    sc = gen.standard_normal((1, 1, 1, cap)).astype(np.float32)
    lens = np.array([cap], dtype=np.int32)
    n = cap - tail
    perm = gen.permutation(n)
    moved = sc.copy()
    moved[0, 0, 0, perm] = sc[0, 0, 0, :n]  # score of cell c now sits at perm[c]
    a = oracle.topk(sc, lens, k, tail, lib=lib)[0, 0, 0, :k]
    b = oracle.topk(moved, lens, k, tail, lib=lib)[0, 0, 0, :k]
    return float(not np.array_equal(np.sort(perm[a]), b))


ALL_CHECKS = {
    "sdpa_dense": check_sdpa_dense,
    "sdpa_mask": check_sdpa_mask,
    "sdpa_wide_heads": check_sdpa_wide_heads,
    "python_bruteforce": check_python_bruteforce,
    "sdpa_gather": check_sdpa_gather,
    "duplicates": check_duplicates,
    "closed_forms": check_closed_forms,
    "split_invariance": check_split_invariance,
    "causal_rows": check_causal_rows,
    "head_permutation": check_head_permutation,
    "sdpa_steps": check_sdpa_steps,
    "steps_closed_forms": check_steps_closed_forms,
    "q8_quantize": check_q8_quantize,
    "q8_sdpa": check_q8_sdpa,
    "q8_page_permutation": check_q8_page_permutation,
    "q8_append": check_q8_append,
    "topk_brute_force": check_topk_brute_force,
    "topk_closed_forms": check_topk_closed_forms,
    "topk_permutation": check_topk_permutation,
}
