"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, plans launches by its documented rules, and rejects bad
arguments before any HIP call (so no GPU is needed here)."""
import ctypes
import os
import re

import pytest

import decode_attention_flash_amd as ck

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ck_decode_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ck_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(ck.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(ck.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    L = ck.lib()
    for code, text in ck.STATUS.items():
        assert L.ck_status_string(code).decode() == text


def test_plan_merge_slices():
    """About 16 KiB of partials per merge slice, at most 16 slices (each
    beyond the first is a helper polling the unit's arrival count)."""
    assert ck.plan(shape(), num_cus=256)["slices"] == 16            # 4 rows x 64 splits x 256 cols: 256 KiB
    assert ck.plan(shape(n_q=3), num_cus=256)["slices"] == 16       # 12 rows: 48 by size, capped
    assert ck.plan(shape(n_q=6), num_cus=256)["slices"] == 16       # two 16-row groups
    assert ck.plan(shape(Hq=8, Hkv=2, D=128, cap=1024), num_cus=256)["slices"] == 2  # 16 x 4 x 128: 32 KiB
    assert ck.plan(shape(B=32, Hq=32, Hkv=8, D=128, cap=32768), num_cus=256)["slices"] == 1  # 8 x 4 x 128
    assert ck.plan(shape(), num_splits=1, num_cus=256)["slices"] == 1


def test_contraction_choice():
    """Only the two documented contractions are accepted; the default is
    restored afterwards."""
    with pytest.raises(ValueError):
        ck.set_contraction("sparse")
    L = ck.lib()
    assert L.ck_set_contraction(3) == -1 and L.ck_set_contraction(-1) == -1
    for kind in ("valu", "valu_f32", "mfma"):
        ck.set_contraction(kind)


def test_phase_stamps_arguments():
    L = ck.lib()
    assert L.ck_set_phase_stamps(None, 5) == -1
    assert L.ck_set_phase_stamps(ctypes.c_void_p(4096), 0) == -1
    assert L.ck_set_phase_stamps(ctypes.c_void_p(4096), -1) == -1
    assert L.ck_set_phase_stamps(ctypes.c_void_p(4100), 3) == -3  # CK_ERR_ALIGN, nothing is written
    assert L.ck_set_phase_stamps(None, 0) == 0


def shape(B=1, n_q=1, Hq=16, Hkv=4, D=256, cap=24007):
    return ck.Shape(B, n_q, Hq, Hkv, D, cap)


def test_plan_fills_the_chip_at_batch_one():
    p = ck.plan(shape(), num_cus=256)
    assert p["units"] == 4 and p["split_target"] == 64 and p["splits"] == 64
    assert p["rows"] == 4 and p["rows_per_group"] == 16 and p["row_groups"] == 1
    assert p["workspace_bytes"] > 0


@pytest.mark.parametrize("B,Hkv,n_q,W", [(3, 4, 1, 0), (1, 2, 6, 4160), (5, 8, 1, 0), (1, 4, 5, 2112)])
def test_plan_keeps_workgroups_in_one_round(B, Hkv, n_q, W):
    # unit counts that do not divide the CU count: the split target rounds
    # down, so units x splits never exceeds one workgroup per CU
    p = ck.plan(shape(B=B, Hq=4 * Hkv, Hkv=Hkv, n_q=n_q, D=128, cap=65536), W=W, num_cus=256)
    assert p["units"] * p["split_target"] <= 256
    assert p["units"] * (p["split_target"] + 1) > 256
    assert p["units"] * p["splits"] <= 256


@pytest.mark.parametrize("B,D,Hq,Hkv,n_q,tile", [
    (1, 128, 8, 2, 1, 32),    # up to 16 packed rows: 8 KiB tiles, two workgroups per CU
    (1, 128, 16, 2, 3, 32),   # 24 rows as two 16-row groups, 64 splits each
    (8, 128, 16, 2, 3, 64),   # 24 rows, 8 splits at most: one group, two row tiles, 16 KiB tiles
    (1, 256, 16, 4, 1, 16),   # 8 KiB: 16 tokens, PV in 16-token k-blocks
    (1, 256, 16, 4, 6, 16),   # 24 rows as two 16-row groups
    (8, 256, 16, 4, 6, 32),   # 24 rows in one group: 16 KiB
])
def test_plan_reports_the_kernel_tile(B, D, Hq, Hkv, n_q, tile):
    p = ck.plan(shape(B=B, n_q=n_q, Hq=Hq, Hkv=Hkv, D=D), num_cus=256)
    assert p["tile"] == tile and p["granule"] % p["tile"] == 0


def test_plan_single_sequence_has_no_chunk_limit():
    p = ck.plan(shape(), num_cus=256)
    assert p["chunk_max"] == 0


def test_plan_does_not_depend_on_capacity_for_split_target():
    a = ck.plan(shape(cap=8199), num_cus=256)
    b = ck.plan(shape(cap=24007), num_cus=256)
    assert a["split_target"] == b["split_target"] and a["chunk_max"] == b["chunk_max"]
    assert a["granule"] == b["granule"]


def test_plan_batched_uses_chunk_limit():
    p = ck.plan(shape(B=32, Hq=32, Hkv=8, D=128, cap=32768), num_cus=256)
    assert p["units"] == 256 and p["split_target"] == 1
    assert p["chunk_max"] == 4096 and p["splits"] == 8


def test_plan_minimum_range_grows_with_rows():
    # at least 5 tokens per packed row, in whole tiles
    assert ck.plan(shape(), num_cus=256)["chunk_min"] == 32
    assert ck.plan(shape(n_q=3), num_cus=256)["chunk_min"] == 64
    assert ck.plan(shape(n_q=6), num_cus=256)["chunk_min"] == 96  # 16-row groups
    assert ck.plan(shape(B=8, n_q=6), num_cus=256)["chunk_min"] == 128  # one 24-row group
    assert ck.plan(shape(B=32, Hq=32, Hkv=8, D=128, cap=32768), num_cus=256)["chunk_min"] == 64
    # a forced split count is used as given
    assert ck.plan(shape(n_q=6), num_splits=64, num_cus=256)["chunk_min"] == 32


def test_plan_causal_window_row_groups():
    # 17-32 packed rows: two 16-row groups while each keeps at least 16
    # splits, else one 32-row group; more than 32 rows: 16-row groups
    p = ck.plan(shape(n_q=6), num_cus=256)
    assert p["rows"] == 24 and p["rows_per_group"] == 16 and p["row_groups"] == 2 and p["units"] == 8
    p = ck.plan(shape(n_q=6, Hq=32, Hkv=4), num_cus=256)  # 48 rows -> three groups
    assert p["rows"] == 48 and p["rows_per_group"] == 16 and p["row_groups"] == 3 and p["units"] == 12
    p = ck.plan(shape(B=4, n_q=6), num_cus=256)  # 32 units of 16 rows: 8 splits
    assert p["rows_per_group"] == 32 and p["row_groups"] == 1 and p["units"] == 16
    p = ck.plan(shape(B=8, n_q=6, Hq=32, Hkv=4), num_cus=256)
    assert p["rows"] == 48 and p["rows_per_group"] == 16 and p["row_groups"] == 3 and p["units"] == 96
    p = ck.plan(shape(B=2, n_q=6), num_cus=256)  # 16 units of 16 rows: 16 splits each
    assert p["rows_per_group"] == 16 and p["row_groups"] == 2 and p["units"] == 16
    p = ck.plan(shape(n_q=6), num_cus=64)  # a smaller chip: 8 units of 16 rows would get 8 splits
    assert p["rows_per_group"] == 32 and p["row_groups"] == 1
    p = ck.plan(shape(Hq=128, Hkv=4), num_cus=256)  # 32-wide GQA groups, one query
    assert p["rows"] == 32 and p["rows_per_group"] == 16 and p["row_groups"] == 2


def test_plan_gather_units_per_query():
    p = ck.plan(shape(Hq=16, Hkv=2, D=128, cap=131072, n_q=2), W=2112, num_cus=256)
    assert p["rows"] == 8 and p["units"] == 4
    assert p["splits"] <= (2112 + 63) // 64


def test_plan_forced_splits_and_single_split():
    p = ck.plan(shape(), num_splits=7, num_cus=256)
    assert p["splits"] == 7 and p["chunk_max"] == 0
    p = ck.plan(shape(), num_splits=1, num_cus=256)
    assert p["splits"] == 1 and p["workspace_bytes"] == 0
    p = ck.plan(shape(cap=10), num_cus=256)  # one tile at most
    assert p["splits"] == 1 and p["workspace_bytes"] == 0


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), -2), (dict(D=129), -2), (dict(n_q=7), -2), (dict(n_q=0), -1),
    (dict(Hq=6, Hkv=4), -1), (dict(B=0), -1), (dict(cap=0), -1),
    (dict(Hkv=8, Hq=8, D=256, cap=600000), -2),
])
def test_plan_rejects(kw, status):
    p = ck.Plan()
    st = ck.lib().ck_decode_attn_plan(ctypes.byref(shape(**kw)), 0, 0, 256, ctypes.byref(p))
    assert st == status


def _call_dense(sh, q=16, k=16, v=16, lens=16, out=16, out_dtype=0, scale=0.1, num_splits=0,
                lse=None):
    V = lambda x: None if x is None else ctypes.c_void_p(x)
    return ck.lib().ck_decode_attn(ctypes.byref(sh), V(q), V(k), V(v), V(lens),
                                   ctypes.c_float(scale), 0, None, V(out), out_dtype, V(lse),
                                   None, 0, num_splits, None)


def test_dense_argument_errors_before_any_hip_call():
    sh = shape()
    big = 1 << 20
    assert _call_dense(sh, q=None) == -1
    assert _call_dense(sh, out=None) == -1
    assert _call_dense(sh, lens=None) == -1
    assert _call_dense(sh, out_dtype=7) == -1
    assert _call_dense(sh, scale=float("nan")) == -1
    assert _call_dense(sh, num_splits=-1) == -1
    assert _call_dense(sh, num_splits=257) == -1
    assert _call_dense(sh, q=big + 8) == -3
    assert _call_dense(sh, out=big + 4) == -3
    assert _call_dense(sh, lens=big + 2) == -3
    assert _call_dense(sh, lse=big + 1) == -3
    assert _call_dense(shape(D=64)) == -2
    assert ck.lib().ck_decode_attn(None, None, None, None, None, ctypes.c_float(1.0), 0, None,
                                   None, 0, None, None, 0, 0, None) == -1


def test_gather_argument_errors_before_any_hip_call():
    sh = shape(Hkv=2, D=128, cap=4096)
    V = ctypes.c_void_p
    L = ck.lib()
    args = lambda W, idx, hs: (ctypes.byref(sh), V(16), V(16), V(16), V(16), idx, W, hs,
                               ctypes.c_float(0.1), 0, V(16), 0, None, None, 0, 0, None)
    assert L.ck_decode_attn_gather(*args(0, V(16), 0)) == -1          # W < 1
    assert L.ck_decode_attn_gather(*args(64, None, 0)) == -1          # no list
    assert L.ck_decode_attn_gather(*args(64, V(16), 10)) == -1        # head stride < W
    assert L.ck_decode_attn_gather(*args(64, V(18), 64)) == -3        # misaligned list


def test_workspace_size_rejects_bad_shape():
    n = ctypes.c_size_t(0)
    assert ck.lib().ck_decode_attn_workspace_size(ctypes.byref(shape(D=64)), 0, 0,
                                                   ctypes.byref(n)) == -2
    assert ck.lib().ck_decode_attn_workspace_size(ctypes.byref(shape()), 0, 0, None) == -1


def _q8(page=64, max_pages=4, num_pages=8, codes=0x10000, scales=0x20000, table=0x30000):
    return ck.Q8CacheC(codes, codes + 0x1000000, scales, scales + 0x1000000, table, page, max_pages, num_pages)


@pytest.mark.parametrize("kw,status", [
    (dict(page=48), -1), (dict(page=0), -1), (dict(max_pages=0), -1), (dict(num_pages=0), -1),
    (dict(codes=0), -1), (dict(table=0), -1), (dict(codes=0x10008), -3), (dict(scales=0x20002), -3),
])
def test_q8_attention_rejects_bad_cache(kw, status):
    """Checked on the host before any HIP call (pointers are never read)."""
    c = _q8(**kw)
    sh = shape(cap=c.page_tokens * c.max_pages)
    st = ck.lib().ck_decode_attn_q8(ctypes.byref(sh), ctypes.c_void_p(0x40000), ctypes.byref(c),
                                    ctypes.c_void_p(0x50000), ctypes.c_float(0.1), 0, ctypes.c_void_p(0x60000),
                                    0, None, None, 0, 0, None)
    assert st == status


def test_q8_attention_capacity_must_match_pages():
    c = _q8()
    sh = shape(cap=c.page_tokens * c.max_pages + 1)
    st = ck.lib().ck_decode_attn_q8(ctypes.byref(sh), ctypes.c_void_p(0x40000), ctypes.byref(c),
                                    ctypes.c_void_p(0x50000), ctypes.c_float(0.1), 0, ctypes.c_void_p(0x60000),
                                    0, None, None, 0, 0, None)
    assert st == -1


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), -2), (dict(n_q=0), -1), (dict(cap=100), -1), (dict(start=0), -1), (dict(start=0x50002), -3),
])
def test_q8_append_rejects(kw, status):
    c = _q8()
    start = kw.pop("start", 0x50000)
    sh = shape(**{"cap": c.page_tokens * c.max_pages, **kw})
    st = ck.lib().ck_kv_append_q8(ctypes.byref(sh), ctypes.c_void_p(0x40000), ctypes.c_void_p(0x48000),
                                  ctypes.c_void_p(start) if start else None, ctypes.byref(c), None)
    assert st == status


# ------------------------------------------------ gather-vs-scan choice ----

@pytest.mark.parametrize("D,Hkv,n_q,W,n_kv,want", [
    (128, 2, 1, 2112, 131072, "gather"),   # the sparse workload: lists far shorter than the window
    (128, 2, 6, 2048, 2048, "gather"),     # short window, the scan's fixed cost: measured 10.0 vs 11.0 us
    (128, 2, 1, 32768, 32768, "gather"),   # whole window listed once: measured 14.6 vs 15.2 us
    (128, 2, 3, 32768, 32768, "scan"),     # listed three times: measured 23.9 vs 18.1 us
    (128, 2, 6, 32768, 32768, "scan"),     # measured 33.0 vs 21.8 us
    (256, 4, 6, 1024, 8192, "gather"),     # measured 12.1 vs 18.2 us
    (256, 4, 6, 4096, 8192, "scan"),       # measured 21.4 vs 18.2 us
    (256, 4, 3, 4096, 32768, "gather"),    # measured 16.8 vs 30.5 us
    (256, 4, 3, 16384, 32768, "scan"),     # measured 39.5 vs 30.5 us
])
def test_sparse_path_follows_measurements(D, Hkv, n_q, W, n_kv, want):
    s = shape(B=1, n_q=n_q, Hq=4 * Hkv, Hkv=Hkv, D=D, cap=max(n_kv, 1))
    assert ck.sparse_path(s, W, n_kv) == want


def test_sparse_path_switches_once_as_lists_grow():
    # more listed cells only make the gather costlier: once the scan wins it keeps winning
    for D, Hkv, n_q, n_kv in ((128, 2, 1, 65536), (128, 2, 6, 16384), (256, 4, 3, 8192)):
        s = shape(n_q=n_q, Hq=4 * Hkv, Hkv=Hkv, D=D, cap=n_kv)
        picks = [ck.sparse_path(s, W, n_kv) for W in range(64, 4 * n_kv + 1, 64)]
        flips = sum(1 for a, b in zip(picks, picks[1:]) if a != b)
        assert flips <= 1 and picks[0] == "gather"


def test_sparse_path_ignores_capacity():
    a = ck.sparse_path(shape(cap=8199), 2112, 8000)
    b = ck.sparse_path(shape(cap=24007), 2112, 8000)
    assert a == b


@pytest.mark.parametrize("kw,W,n_kv,status", [
    (dict(), 0, 1000, -1), (dict(), 64, -1, -1), (dict(D=64), 64, 1000, -2), (dict(n_q=7), 64, 1000, -2),
])
def test_sparse_path_rejects(kw, W, n_kv, status):
    path = ctypes.c_int32(-7)
    st = ck.lib().ck_decode_sparse_path(ctypes.byref(shape(**kw)), W, n_kv, ctypes.byref(path))
    assert st == status and path.value == -7
    assert ck.lib().ck_decode_sparse_path(ctypes.byref(shape()), 64, 1000, None) == -1


# ----------------------------------------------------------------- top-k ----

@pytest.mark.parametrize("B,n_q,Hs,cap,cus", [(1, 1, 2, 131072, 256), (1, 3, 4, 24007, 256), (32, 1, 8, 32768, 256),
                                              (2, 1, 1, 3000, 256), (1, 1, 1, 500, 256), (7, 2, 3, 65536, 80)])
def test_topk_plan_keeps_row_workgroups_resident(B, n_q, Hs, cap, cus):
    p = ck.topk_plan((B, n_q, Hs, cap), k=2048, tail=64, num_cus=cus)
    rows = B * n_q * Hs
    P = p["wgs_per_row"]
    assert 1 <= P <= 256 and P <= (cap + 4095) // 4096  # at least 4096 positions per workgroup
    if P > 1:  # a row's workgroups wait for each other: all must fit at once
        assert rows * P <= cus and p["workspace_bytes"] > 0
    else:
        assert p["workspace_bytes"] == 0
    if rows >= cus:
        assert P == 1


@pytest.mark.parametrize("scores_shape,kw,status", [
    ((1, 1, 3, 1000), dict(k=10, num_kv_heads=2), -1),  # score heads neither 1 nor Hkv
    ((1, 1, 2, 1000), dict(k=0), -1),
    ((1, 1, 2, 1000), dict(k=10, tail=-1), -1),
    ((1, 7, 2, 1000), dict(k=10), -2),
    ((0, 1, 2, 1000), dict(k=10), -1),
    ((1, 1, 1, 1 << 28), dict(k=10), -2),  # one row's pair slots would pass 2 GiB (32-bit offsets)
])
def test_topk_plan_rejects(scores_shape, kw, status):
    with pytest.raises(ck.CkError) as e:
        ck.topk_plan(scores_shape, num_cus=256, **kw)
    assert e.value.status == status


def test_topk_plan_largest_rows():
    # 2^27 positions in one row: 256 workgroups, 1 GiB of pair slots
    p = ck.topk_plan((1, 1, 1, 1 << 27), k=2048, tail=64, num_cus=256)
    assert p["wgs_per_row"] == 256 and p["workspace_bytes"] > (1 << 30)


def test_topk_entry_rejects_before_launch():
    # argument errors come back before any HIP call (no GPU here)
    s = ck.Shape(1, 1, 2, 2, 128, 1000)
    L = ck.lib()
    assert L.ck_decode_topk(ctypes.byref(s), None, 2, None, 10, 0, 0, None, None, 0, None) == -1
    assert L.ck_decode_topk(ctypes.byref(s), ctypes.c_void_p(16), 3, ctypes.c_void_p(16), 10, 0, 0,
                            ctypes.c_void_p(16), None, 0, None) == -1
    assert L.ck_decode_topk(ctypes.byref(s), ctypes.c_void_p(18), 2, ctypes.c_void_p(16), 10, 0, 0,
                            ctypes.c_void_p(16), None, 0, None) == -3
