"""GPU: top-k index lists (ck_decode_topk) against the oracle, bit-exact.

Covers the sparse workload's shape (two score rows of 131072 cells, many
workgroups per row meeting at barriers), rows full of ties and special
values, causal windows, one workgroup per row (a large batch), unaligned
score rows, workspace reuse across calls and graph replays, and the lists
feeding the gather."""
import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
import oracle
from decode_attention_flash_amd import synth
from gpu_common import DEV, assert_close, gather_gpu, note, oracle_ref

pytestmark = pytest.mark.gpu


def topk_gpu(scores, lens, k, tail=0, causal=False, num_kv_heads=None):
    out = ck.decode_topk(scores.to(DEV), torch.as_tensor(np.asarray(lens), dtype=torch.int32).to(DEV), k,
                         tail=tail, causal=causal, num_kv_heads=num_kv_heads)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(scores, lens, k, tail=0, causal=False, what=""):
    got = topk_gpu(scores, lens, k, tail, causal)
    ref = oracle.topk(scores.numpy(), np.asarray(lens, dtype=np.int32), k, tail, causal)
    bad = np.argwhere(np.any(got != ref, axis=-1))
    assert bad.size == 0, f"{what}: rows {bad[:4].tolist()} differ"
    return got


@pytest.mark.parametrize("n_kv", [32768, 131072])
def test_sparse_workload_lists(n_kv):
    """Two score rows (one per KV head), 2048 best + the last 64 cells."""
    note(f"topk sparse workload n_kv={n_kv}")
    sc = synth.index_scores(1, 1, 2, n_kv, 7000 + n_kv)
    got = check(sc, [n_kv], 2048, 64, what=f"n_kv={n_kv}")
    assert got.shape == (1, 1, 2, 2112) and np.all(np.diff(got, axis=-1) > 0)


def test_ties_specials_causal_ragged():
    """Small-integer scores (many exact ties), NaN, +-inf and signed zeros;
    three causal queries per sequence; lengths 0, short, long and past the
    capacity (clamped); two score heads."""
    note("topk ties / specials / causal")
    B, n_q, Hs, cap = 4, 3, 2, 20000
    rng = np.random.default_rng(71)
    sc = rng.integers(-4, 5, size=(B, n_q, Hs, cap)).astype(np.float32)
    m = rng.random(sc.shape) < 0.05
    sc[m] = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0], np.float32)[rng.integers(0, 5, int(m.sum()))]
    check(torch.from_numpy(sc), [0, 700, cap, cap + 999], 700, 17, causal=True, what="ties")


def test_all_candidates_and_tiny_windows():
    """k at or above the candidates: every cell before the tail, then the tail."""
    note("topk k >= candidates")
    sc = synth.index_scores(3, 1, 1, 4096, 72)
    check(sc, [1, 64, 4000], 4000, 5, what="k >= n")
    check(sc, [3, 2, 4096], 10, 4, what="windows shorter than the tail")


def test_one_workgroup_per_row():
    """256 rows fill the chip: each row is one workgroup (no barriers), and
    its 8 super-blocks of keys all stay in registers across the passes."""
    note("topk one workgroup per row")
    B, Hs, cap = 32, 8, 32768
    plan = ck.topk_plan((B, 1, Hs, cap), 2048, 64)
    assert plan["wgs_per_row"] == 1
    lens = synth.ragged_lens(B, 512, cap, 4000)
    sc = synth.index_scores(B, 1, Hs, cap, 73)
    check(sc, lens, 2048, 64, what="batch")


@pytest.mark.parametrize("B,Hs,cap", [(32, 8, 40000), (4, 8, 131072), (8, 8, 200000)])
def test_cached_and_reread_super_blocks(B, Hs, cap):
    """Workgroups holding several 4096-cell blocks: one per row with 10
    blocks (8 kept in registers, 2 read again per pass), 8 per row with 4
    blocks each, and 4 per row with 13 blocks each (the cache plus 5 read
    again), on ragged lengths."""
    plan = ck.topk_plan((B, 1, Hs, cap), 2048, 64)
    blocks = -(-cap // 4096)
    per = -(-blocks // plan["wgs_per_row"])
    note(f"topk cached blocks B={B} Hs={Hs} cap={cap} P={plan['wgs_per_row']} blocks/wg={per}")
    assert per > 1
    lens = synth.ragged_lens(B, cap // 2, cap, 75)
    sc = synth.index_scores(B, 1, Hs, cap, 76)
    check(sc, lens, 2048, 64, what=f"cap={cap}")


def test_unaligned_rows_and_shared_lists():
    """cap % 4 != 0 (scores read one at a time) and one score row per query
    shared by the KV heads (Hs = 1)."""
    note("topk unaligned rows")
    sc = synth.index_scores(2, 2, 1, 5003, 74)
    got = topk_gpu(sc, [5003, 4111], 300, 9, causal=True, num_kv_heads=4)
    ref = oracle.topk(sc.numpy(), np.array([5003, 4111], np.int32), 300, 9, True)
    assert np.array_equal(got, ref)


def test_workspace_reuse_and_graph_replay():
    """The workspace is left zeroed: repeated calls with new scores and new
    lengths, eagerly and replayed from a captured graph, all match."""
    note("topk replay")
    B, Hs, cap, k, tail = 1, 2, 65536, 2048, 64
    sc_d = torch.empty((B, 1, Hs, cap), dtype=torch.float32, device=DEV)
    lens_d = torch.empty((B,), dtype=torch.int32, device=DEV)
    out_d = torch.empty((B, 1, Hs, k + tail), dtype=torch.int32, device=DEV)
    cases = [(synth.index_scores(B, 1, Hs, cap, 80 + r), np.array([cap - 977 * r], np.int32)) for r in range(4)]
    for sc, lens in cases:  # eager
        sc_d.copy_(sc)
        lens_d.copy_(torch.from_numpy(lens))
        ck.decode_topk(sc_d, lens_d, k, tail=tail, out=out_d)
        torch.cuda.synchronize()
        assert np.array_equal(out_d.cpu().numpy(), oracle.topk(sc.numpy(), lens, k, tail))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ck.decode_topk(sc_d, lens_d, k, tail=tail, out=out_d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ck.decode_topk(sc_d, lens_d, k, tail=tail, out=out_d)
    for sc, lens in cases:
        sc_d.copy_(sc)
        lens_d.copy_(torch.from_numpy(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_d.cpu().numpy(), oracle.topk(sc.numpy(), lens, k, tail))


def test_lists_feed_the_gather():
    """Selection then gathered attention equals the oracle's attention over
    the oracle's lists."""
    note("topk -> gather")
    B, n_q, Hq, Hkv, D, cap = 1, 3, 16, 2, 128, 32768
    L = 30000
    k, v = synth.kv_cache(B, cap, Hkv, D, [L], 1011)
    q = synth.queries(B, n_q, Hq, D, 1011)
    sc = synth.index_scores(B, n_q, Hkv, cap, 1011)
    lists = topk_gpu(sc, [L], 2048, 64, causal=True)
    ref_lists = oracle.topk(sc.numpy(), np.array([L], np.int32), 2048, 64, True)
    assert np.array_equal(lists, ref_lists)
    gpu = gather_gpu(q, k, v, [L], lists, causal=True)
    assert_close(gpu, oracle_ref(q, k, v, [L], causal=True, idx=ref_lists), what="topk -> gather")


@pytest.mark.parametrize("kind", ["rising", "falling", "flat", "two_values"])
def test_concentrated_and_tied_rows_full_size(kind):
    """Full-size rows (131072 cells, 32 workgroups) where the threshold bin
    sits in one workgroup's range (rising / falling scores), where every
    score ties (flat: the digit-by-digit path with tie ranks spanning all
    workgroups), and two values (a bin too large to gather)."""
    note(f"topk full-size {kind}")
    n_kv = 131072
    cells = torch.arange(n_kv, dtype=torch.float32)
    if kind == "rising":
        row = cells / n_kv
    elif kind == "falling":
        row = -cells / n_kv
    elif kind == "flat":
        row = torch.full((n_kv,), 0.25)
    else:
        row = (torch.arange(n_kv) % 3 == 0).to(torch.float32)
    sc = torch.stack([row, row.flip(0)]).view(1, 1, 2, n_kv).contiguous()
    check(sc, [n_kv], 2048, 64, what=kind)
    check(sc, [n_kv - 12345], 2048, 64, causal=False, what=f"{kind} shorter")


@pytest.mark.parametrize("n_kv", [32768, 131072])
@pytest.mark.parametrize("copies", [30, 62, 70, 300])
def test_threshold_ties_in_lds_selection(n_kv, copies):
    """Normal scores whose k-th largest value is copied into `copies` other
    cells below it: the threshold bin still fits in LDS, and after its
    11-bit digit the remaining bin holds about `copies` keys, so both the
    one-wave ranking (up to 64 keys) and the last histogram level (more)
    choose among exact ties."""
    note(f"topk threshold ties n_kv={n_kv} copies={copies}")
    sc = synth.index_scores(1, 1, 2, n_kv, 7100 + copies).numpy().copy()
    rng = np.random.default_rng(7200 + copies)
    for h in range(2):
        row = sc[0, 0, h, : n_kv - 64]
        v = np.sort(row)[::-1][2047]
        below = np.flatnonzero(row < v)
        row[rng.choice(below, size=copies, replace=False)] = v
    got = check(torch.from_numpy(sc), [n_kv], 2048, 64, what=f"ties {copies}")
    assert np.all(np.diff(got, axis=-1) > 0)
