"""GPU: top-k selections through the masked scan (which skips tiles that
hold no kept cell) and through the gather-or-scan choice.

Skipping must not change which cells are attended: the tests compare with
the oracle, recover exact cell sets with the counting construction (splits
long enough to cross several 64-tile windows of the tile bitmap), and check
that a mask stored where tiles cannot be skipped (rows not 16-byte aligned)
gives the same result.  decode_attn_sparse must run the entry point that
ck_decode_sparse_path names and agree with the oracle either way."""
import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
from decode_attention_flash_amd import synth
from gpu_common import (DEV, TOL_F32, assert_close, check_counts, counting_case, gather_gpu, note,
                        oracle_ref)

pytestmark = pytest.mark.gpu


def masked_gpu(q, k, v, lens, mask, *, causal=False, num_splits=0, offset=0, out_dtype=torch.float32):
    """decode_attn with keep_mask stored `offset` bytes into a fresh allocation
    (offset 0: rows 16-byte aligned when cap % 16 == 0, so tiles are skipped;
    offset 4: aligned to 4 bytes only, so every tile is scanned)."""
    B, n_q, Hkv, cap = mask.shape
    buf = torch.zeros(mask.size + offset, dtype=torch.uint8, device=DEV)
    mask_d = buf[offset:].view(B, n_q, Hkv, cap)
    mask_d.copy_(torch.from_numpy(np.ascontiguousarray(mask)).to(DEV))
    lens_d = torch.as_tensor(np.asarray(lens), dtype=torch.int32).to(DEV)
    out, lse = ck.decode_attn(q.to(DEV), k.to(DEV), v.to(DEV), lens_d, causal=causal, keep_mask=mask_d,
                              return_lse=True, num_splits=num_splits, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def visible_sets(mask, lens, causal):
    """Cells each (sequence, query, KV head) attends: kept and below its limit."""
    B, n_q, Hkv, _ = mask.shape
    sets = []
    for b in range(B):
        L = int(lens[b])
        per_i = []
        for i in range(n_q):
            lim = max(0, min(L, L - n_q + i + 1)) if causal else L
            per_i.append([np.flatnonzero(mask[b, i, g, :lim]) for g in range(Hkv)])
        sets.append(per_i)
    return sets


@pytest.mark.parametrize("D,n_kv", [(128, 32768), (128, 131072), (256, 16384)])
def test_block_selection_matches_oracle_and_gather(D, n_kv):
    """The sparse workload with its 2048 + 64 cells chosen as 32 aligned
    blocks of 64: most tiles hold no kept cell."""
    B, n_q, Hq, Hkv = 1, 1, 16, 2
    note(f"mask skip: block selection D={D} n_kv={n_kv}")
    k, v = synth.kv_cache(B, n_kv, Hkv, D, [n_kv], 1006)
    q = synth.queries(B, n_q, Hq, D, 1006)
    idx = synth.block_lists(B, n_q, Hkv, n_kv, 32, 64, 64, seed=5100 + n_kv)
    mask = synth.mask_from_lists(idx, n_kv)
    masked = masked_gpu(q, k, v, [n_kv], mask)
    assert_close(masked, oracle_ref(q, k, v, [n_kv], keep_mask=mask), what=f"block mask {n_kv}")
    gathered = gather_gpu(q, k, v, [n_kv], idx)
    assert np.max(np.abs(gathered[0] - masked[0])) <= TOL_F32
    assert np.max(np.abs(gathered[1] - masked[1])) <= 4e-3


def crossing_mask(B, n_q, Hkv, cap, lens, seed, TT):
    """Per (sequence, query, head): a few kept runs, scattered single cells in
    otherwise empty tiles, kept cells past the length (never visible), one
    head with nothing kept in range and one with only the last in-range cell."""
    rng = np.random.default_rng(seed)
    m = np.zeros((B, n_q, Hkv, cap), dtype=np.uint8)
    for b in range(B):
        L = int(lens[b])
        for i in range(n_q):
            for g in range(Hkv):
                case = (b + i + g) % 5
                if case == 0:  # nothing kept before the length
                    m[b, i, g, L:] = 1
                    continue
                if case == 1:  # only the last cell of the sequence
                    m[b, i, g, L - 1] = 1
                    continue
                for _ in range(4):  # runs of one to three tiles
                    s = int(rng.integers(0, max(1, L // TT))) * TT
                    m[b, i, g, s:s + TT * int(rng.integers(1, 4))] = rng.integers(1, 256)
                cells = rng.integers(0, L, size=7)
                m[b, i, g, cells] = 1
                m[b, i, g, L:L + 5] = 1
    return m


@pytest.mark.parametrize("D,L,splits", [(128, 20000, 1), (128, 20000, 3), (256, 9000, 1), (256, 9000, 2)])
def test_window_crossings_recover_exact_cell_sets(D, L, splits):
    """Splits of 100-300 tiles, so each wave walks several 64-tile windows of
    the bitmap; three causal queries with their own masks; each output
    recovers exactly its visible cell set (counting construction)."""
    n_q, Hq, Hkv = 3, 8, 2
    lens = [L, L // 3 + 11]
    cap = ((L + 40) // 16) * 16
    TT = ck.plan(ck.Shape(len(lens), n_q, Hq, Hkv, D, cap))["tile"]  # the kernel's tile
    note(f"mask skip: window crossings D={D} L={L} splits={splits}")
    q, k, v = counting_case(n_q, Hq, Hkv, D, cap, lens, 13)
    mask = crossing_mask(len(lens), n_q, Hkv, cap, lens, 14 + D, TT)
    out, lse = masked_gpu(q, k, v, lens, mask, causal=True, num_splits=splits)
    sets = visible_sets(mask, lens, True)
    check_counts(out, sets, Hq // Hkv)
    for b in range(len(lens)):
        for i in range(n_q):
            for h in range(Hq):
                assert np.isneginf(lse[b, i, h]) == (len(sets[b][i][h // (Hq // Hkv)]) == 0)


@pytest.mark.parametrize("n_q", [3, 6])
def test_mtp_window_with_per_query_block_masks(n_q):
    """Causal verification window, each query with its own block selection:
    a tile is skipped only when no query of the workgroup keeps a cell in it."""
    B, Hq, Hkv, D, L, cap = 1, 16, 4, 256, 4000, 4096
    note(f"mask skip: MTP n_q={n_q}")
    k, v = synth.kv_cache(B, cap, Hkv, D, [L], 1007)
    q = synth.queries(B, n_q, Hq, D, 1007)
    idx = synth.block_lists(B, n_q, Hkv, L, 8, 64, 16, seed=5200 + n_q)
    mask = synth.mask_from_lists(idx, cap)
    for out_dtype in (torch.float32, torch.bfloat16):
        gpu = masked_gpu(q, k, v, [L], mask, causal=True, out_dtype=out_dtype)
        assert_close(gpu, oracle_ref(q, k, v, [L], causal=True, keep_mask=mask), out_dtype,
                     what=f"MTP mask n_q={n_q}")


def test_mtp_window_masks_one_32_row_group():
    """A batch of verification windows (24 packed rows on 16 sequence x KV
    head pairs: one 32-row group, two row tiles) with per-query block masks
    and ragged lengths."""
    B, n_q, Hq, Hkv, D, cap = 4, 6, 16, 4, 256, 4096
    lens = [4000, 2500, 1, 3999]
    p = ck.plan(ck.Shape(B, n_q, Hq, Hkv, D, cap))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert p["rows_per_group"] == 32
    note("mask skip: MTP batch, one 32-row group")
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 1011)
    q = synth.queries(B, n_q, Hq, D, 1011)
    idx = synth.block_lists(B, n_q, Hkv, 4000, 8, 64, 16, seed=5500)
    mask = synth.mask_from_lists(idx, cap)
    gpu = masked_gpu(q, k, v, lens, mask, causal=True)
    assert_close(gpu, oracle_ref(q, k, v, lens, causal=True, keep_mask=mask), what="MTP batch mask")


def test_all_masked_rows_are_empty():
    """No kept cell anywhere in range: every split skips all its tiles; the
    output is 0 and the lse -inf."""
    B, n_q, Hq, Hkv, D, cap = 2, 2, 8, 2, 128, 8192
    lens = [8000, 300]
    note("mask skip: all masked")
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 1008)
    q = synth.queries(B, n_q, Hq, D, 1008)
    mask = np.zeros((B, n_q, Hkv, cap), dtype=np.uint8)
    mask[0, :, :, 8000:] = 1  # past the length only
    out, lse = masked_gpu(q, k, v, lens, mask, causal=True)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("D", [128, 256])
def test_skipping_and_full_scan_agree(D):
    """The same masks stored 16-byte aligned (tiles skipped) and 4-byte
    aligned (every tile scanned).  With a kept cell in every tile both take
    the same tiles in the same order: bit-identical.  With block selections
    the waves share the kept tiles differently: equal to rounding."""
    B, n_q, Hq, Hkv, cap = 1, 1, 16, 2, 24576
    TT = ck.plan(ck.Shape(B, n_q, Hq, Hkv, D, cap))["tile"]  # the kernel's tile
    L = 24000
    note(f"mask skip: aligned vs unaligned D={D}")
    k, v = synth.kv_cache(B, cap, Hkv, D, [L], 1009)
    q = synth.queries(B, n_q, Hq, D, 1009)
    rng = np.random.default_rng(1009)
    dense_mask = (rng.random((B, n_q, Hkv, cap)) < 0.3).astype(np.uint8)
    dense_mask[..., ::TT] = 1
    a = masked_gpu(q, k, v, [L], dense_mask, offset=0)
    u = masked_gpu(q, k, v, [L], dense_mask, offset=4)
    assert np.array_equal(a[0], u[0]) and np.array_equal(a[1], u[1])
    idx = synth.block_lists(B, n_q, Hkv, L, 24, 64, 64, seed=5300 + D)
    block_mask = synth.mask_from_lists(idx, cap)
    a = masked_gpu(q, k, v, [L], block_mask, offset=0)
    u = masked_gpu(q, k, v, [L], block_mask, offset=4)
    ref = oracle_ref(q, k, v, [L], keep_mask=block_mask)
    assert_close(a, ref, what="skipping")
    assert_close(u, ref, what="full scan")
    assert np.max(np.abs(a[0] - u[0])) <= 2e-3


@pytest.mark.parametrize("D,Hkv,n_q,W,n_kv,want", [
    (128, 2, 1, 2112, 8192, "gather"),
    (256, 4, 3, 8192, 8192, "scan"),
])
def test_sparse_dispatch_routes_and_matches_oracle(D, Hkv, n_q, W, n_kv, want, monkeypatch):
    B, Hq = 1, 4 * Hkv
    note(f"sparse dispatch D={D} n_q={n_q} W={W} n_kv={n_kv}")
    k, v = synth.kv_cache(B, n_kv, Hkv, D, [n_kv], 1010)
    q = synth.queries(B, n_q, Hq, D, 1010)
    idx = synth.topk_lists(B, n_q, Hkv, n_kv, W - 64, 64, seed=5400 + W)
    mask = synth.mask_from_lists(idx, n_kv)
    calls = []
    scan, gather = ck.decode_attn, ck.decode_attn_gather
    monkeypatch.setattr(ck, "decode_attn", lambda *a, **kw: calls.append("scan") or scan(*a, **kw))
    monkeypatch.setattr(ck, "decode_attn_gather", lambda *a, **kw: calls.append("gather") or gather(*a, **kw))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lens_d = torch.tensor([n_kv], dtype=torch.int32, device=DEV)
    idx_d = torch.from_numpy(idx).to(DEV)
    mask_d = torch.from_numpy(mask).to(DEV)
    causal = n_q > 1
    ref = oracle_ref(q, k, v, [n_kv], causal=causal, keep_mask=mask)
    out, lse = ck.decode_attn_sparse(qd, kd, vd, lens_d, idx_d, keep_mask=mask_d, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert calls == [want]
    assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what=f"sparse {want}")
    calls.clear()  # without a mask only the gather can serve
    out, lse = ck.decode_attn_sparse(qd, kd, vd, lens_d, idx_d, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert calls == ["gather"]
    assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what="sparse without mask")


@pytest.mark.parametrize("D,n_q,causal,offset", [(128, 1, False, 0), (128, 1, False, 4), (256, 1, False, 0),
                                                 (128, 3, True, 0), (256, 3, False, 4)])
def test_unkept_cells_may_hold_any_bits(D, n_q, causal, offset):
    """Cells below the length that keep_mask excludes for every query of the
    KV head are staged as zeros, so they may hold any bits: with NaN, +-Inf
    and huge values in K and V there, the result equals the oracle's (which
    never reads them) and is bit-identical to the same launch with those
    cells zeroed.  Tiles are skipped (rows 16-byte aligned) or all scanned
    (offset 4)."""
    B, Hq, Hkv, cap = 2, 16, 4, 4096
    lens = [3000, 1777]
    p = ck.plan(ck.Shape(B, n_q, Hq, Hkv, D, cap))
    assert p["rows_per_group"] == 16
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 4100 + D + n_q)
    q = synth.queries(B, n_q, Hq, D, 4101)
    rng = np.random.default_rng(4102 + D + n_q)
    # runs of kept cells (some tiles empty, some partly kept), per query
    mask = np.zeros((B, n_q, Hkv, cap), np.uint8)
    for b in range(B):
        for i in range(n_q):
            for g in range(Hkv):
                starts = rng.choice(cap, size=40, replace=False)
                for s0 in starts:
                    mask[b, i, g, s0:s0 + int(rng.integers(1, 24))] = 1
    unkept = ~mask.any(axis=1)                                  # [B, Hkv, cap]
    bad = np.array([np.nan, np.inf, -np.inf, 3e38], np.float32)
    kz, vz = k.clone(), v.clone()
    kg, vg = k.clone(), v.clone()
    for b in range(B):
        for g in range(Hkv):
            cells = np.flatnonzero(unkept[b, g, :lens[b]])
            kz[b, cells, g] = 0
            vz[b, cells, g] = 0
            fill = torch.from_numpy(bad[rng.integers(0, 4, size=(len(cells), D))]).to(torch.bfloat16)
            kg[b, cells, g] = fill
            vg[b, cells, g] = fill.flip(0)
    note(f"unkept cells hold any bits D={D} n_q={n_q} causal={causal} offset={offset}")
    got = masked_gpu(q, kg, vg, lens, mask, causal=causal, offset=offset)
    zero = masked_gpu(q, kz, vz, lens, mask, causal=causal, offset=offset)
    assert np.array_equal(got[0], zero[0]) and np.array_equal(got[1], zero[1])
    assert_close(got, oracle_ref(q, k, v, lens, causal=causal, keep_mask=mask), what="unkept cells")
