"""GPU parity: the HIP library against the fp64 oracle on the same seeded
inputs, for every decode workload shape, plus the exactness properties
(garbage and capacity invariance, bit-exact index and mask handling)."""

import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
from decode_attention_flash_amd import synth
from gpu_common import (DEV, TOL_F32, assert_close, check_counts, counters_ready, counting_case, dense_gpu,
                        gather_gpu, note, oracle_ref, steps_gpu, steps_ref)

pytestmark = pytest.mark.gpu


# ------------------------------------------------ workload configurations ----

@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_dense(out_dtype):
    """B=1, Hq=8, Hkv=2, D=128, one query, capacity 1024, 300 filled, garbage after."""
    note(f"tiny dense {out_dtype}")
    B, n_q, Hq, Hkv, D, cap, L = 1, 1, 8, 2, 128, 1024, 300
    k, v = synth.kv_cache(B, cap, Hkv, D, [L], 1001)
    q = synth.queries(B, n_q, Hq, D, 1001)
    gpu = dense_gpu(q, k, v, [L], out_dtype=out_dtype)
    assert_close(gpu, oracle_ref(q, k, v, [L]), out_dtype, "tiny")


@pytest.fixture(scope="module")
def layer_d256():
    """Hq=16, Hkv=4, D=256 layer with capacity 24007 filled to 24000."""
    B, Hq, Hkv, D, cap = 1, 16, 4, 256, 24007
    k, v = synth.kv_cache(B, cap, Hkv, D, [24000], 1002)
    return k, v, (k.to(DEV), v.to(DEV))


@pytest.mark.parametrize("L", [1000, 3000, 8000, 24000])
def test_d256_kv_len_sweep(layer_d256, L):
    note(f"D=256 plain decode L={L}")
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, 1, 16, 256, 1002)
    gpu = dense_gpu(q, k, v, [L], device_inputs=(q.to(DEV), kd, vd))
    assert_close(gpu, oracle_ref(q, k, v, [L]), what=f"L={L}")


def test_d256_capacity_sweep_bit_identical():
    """kv_len 3000 at capacities 8199, 16263, 24007: same filled prefix,
    different garbage after it; the outputs are bit-identical."""
    q = synth.queries(1, 1, 16, 256, 1002)
    outs = []
    for cap in (8199, 16263, 24007):
        note(f"capacity sweep cap={cap}")
        k, v = synth.kv_cache(1, cap, 4, 256, [3000], 1002 + cap)
        k[:, :3000], v[:, :3000] = synth.kv_cache(1, 3000, 4, 256, [3000], 1002)
        gpu = dense_gpu(q, k, v, [3000])
        outs.append(gpu)
    ref = oracle_ref(q, k, v, [3000])
    assert_close(outs[0], ref, what="cap sweep")
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])


@pytest.mark.parametrize("n_q", [3, 4, 5, 6])
@pytest.mark.parametrize("L", [2000, 4000, 6144, 6145])  # 6144: the last span with the window split cap
def test_d256_causal_window(layer_d256, n_q, L):
    note(f"causal window n_q={n_q} L={L}")
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, n_q, 16, 256, 1003 + n_q)
    gpu = dense_gpu(q, k, v, [L], causal=True, device_inputs=(q.to(DEV), kd, vd))
    assert_close(gpu, oracle_ref(q, k, v, [L], causal=True), what=f"n_q={n_q} L={L}")


def test_d256_causal_window_bf16_out(layer_d256):
    note("causal window bf16 out")
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, 5, 16, 256, 1013)
    gpu = dense_gpu(q, k, v, [2000], causal=True, out_dtype=torch.bfloat16,
                    device_inputs=(q.to(DEV), kd, vd))
    assert_close(gpu, oracle_ref(q, k, v, [2000], causal=True), torch.bfloat16, "bf16 window")


def test_causal_rows_equal_shorter_plain_decode(layer_d256):
    """Causal row i equals a single-query decode of length L - n_q + i + 1."""
    k, v, (kd, vd) = layer_d256
    n_q, L = 6, 4000
    q = synth.queries(1, n_q, 16, 256, 1023)
    note("causal rows vs plain")
    full, _ = dense_gpu(q, k, v, [L], causal=True, device_inputs=(q.to(DEV), kd, vd))
    for i in range(n_q):
        qi = q[:, i:i + 1].contiguous()
        row, _ = dense_gpu(qi, k, v, [L - n_q + i + 1], device_inputs=(qi.to(DEV), kd, vd))
        assert np.max(np.abs(row[:, 0] - full[:, i])) <= TOL_F32


# ------------------------------------------------------------- batched ----

def test_batched_ragged_graph_replay():
    """B=32, Hq=32, Hkv=8, D=128, capacity 32768, lengths uniform in
    [512, 32768]; one captured launch replayed with new lengths each time."""
    B, Hq, Hkv, D, cap = 32, 32, 8, 128, 32768
    note("batched ragged: generating caches on the device")
    k, v = synth.kv_cache(B, cap, Hkv, D, [cap] * B, 1004, device=DEV, garbage=False)
    q = synth.queries(B, 1, Hq, D, 1004, device=DEV)
    lens_d = torch.zeros(B, dtype=torch.int32, device=DEV)
    shape = ck.shape_of(q, k)
    ws = ck.new_workspace(shape)
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=DEV)
    lens_d.copy_(torch.from_numpy(synth.ragged_lens(B, 512, cap, 3999)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ck.decode_attn(q, k, v, lens_d, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note("batched ragged: capture")
    with torch.cuda.graph(graph):
        ck.decode_attn(q, k, v, lens_d, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    kh, vh, qh = k.cpu(), v.cpu(), q.cpu()  # the same bytes for the oracle (4 GiB of K+V)
    for r in range(3):
        lens = synth.ragged_lens(B, 512, cap, 4000 + r)
        lens_d.copy_(torch.from_numpy(lens))
        note(f"batched ragged: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        ls = lse.cpu().numpy()
        # eager launch on the same lengths gives the same bits as the replay
        eo, el = ck.decode_attn(q, k, v, lens_d, return_lse=True, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(eo.cpu().numpy(), o) and np.array_equal(el.cpu().numpy(), ls)
        # every sequence of the batch against the oracle
        assert_close((o, ls), oracle_ref(qh, kh, vh, lens), what=f"replay {r} (all {B} sequences)")
    # the counters are ready for the next launch (the set it will use is zero)
    assert counters_ready(ws, ck.plan(shape)["units"])


# ----------------------------------------------------- step-row merge ----

def _steps(B, n_q, Hkv, D, seed):
    gen = synth.generator(seed)
    return synth.bf16_normal((B, n_q, Hkv, D), gen), synth.bf16_normal((B, n_q, Hkv, D), gen)


@pytest.mark.parametrize("n_q", [1, 3, 6])
@pytest.mark.parametrize("L", [0, 1, 37, 2000, 4000, 6144, 6145])
def test_d256_step_rows_match_oracle(layer_d256, n_q, L):
    """MTP verification with the drafts passed beside the cache: prefix
    [0, L) plus step rows 0..i for query i (bf16 output for the longer
    prefixes)."""
    out_dtype = torch.bfloat16 if L >= 2000 else torch.float32
    note(f"step rows D=256 n_q={n_q} L={L} {out_dtype}")
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, n_q, 16, 256, 1030 + n_q)
    ks, vs = _steps(1, n_q, 4, 256, 1040 + n_q + L)
    gpu = steps_gpu(q, k, v, [L], ks, vs, device_inputs=(q.to(DEV), kd, vd), out_dtype=out_dtype)
    assert_close(gpu, steps_ref(q, k, v, [L], ks, vs), out_dtype, what=f"steps n_q={n_q} L={L}")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_d128_step_rows_batch(out_dtype):
    """Two sequences of different length (one empty), D=128, ragged tail."""
    B, n_q, Hq, Hkv, D, cap = 2, 4, 8, 2, 128, 1024
    lens = [301, 0]
    note(f"step rows D=128 batch {out_dtype}")
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 1050)
    q = synth.queries(B, n_q, Hq, D, 1051)
    ks, vs = _steps(B, n_q, Hkv, D, 1052)
    gpu = steps_gpu(q, k, v, lens, ks, vs, out_dtype=out_dtype)
    assert_close(gpu, steps_ref(q, k, v, lens, ks, vs), out_dtype, "steps D=128")


def test_step_rows_one_32_row_group():
    """24 packed rows on 16 (sequence, KV head) pairs: one 32-row group with
    two row tiles; ragged prefixes, one empty."""
    B, n_q, Hq, Hkv, D, cap = 4, 6, 16, 4, 256, 1600
    lens = [900, 0, 1501, 37]
    p = ck.plan(ck.Shape(B, n_q, Hq, Hkv, D, cap))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert p["rows_per_group"] == 32 and p["row_groups"] == 1
    note("step rows one 32-row group")
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 1060)
    q = synth.queries(B, n_q, Hq, D, 1061)
    ks, vs = _steps(B, n_q, Hkv, D, 1062)
    gpu = steps_gpu(q, k, v, lens, ks, vs)
    assert_close(gpu, steps_ref(q, k, v, lens, ks, vs), what="steps 32-row group")


def test_step_rows_equal_causal_window_in_cache(layer_d256):
    """The same window computed both ways on the GPU: drafts beside the cache,
    and drafts written into the cache at [L, L + n_q) with the causal mask."""
    n_q, L = 5, 3000
    note("step rows vs causal window")
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, n_q, 16, 256, 1060)
    ks, vs = _steps(1, n_q, 4, 256, 1061)
    a = steps_gpu(q, k, v, [L], ks, vs, device_inputs=(q.to(DEV), kd, vd))
    kc, vc = kd.clone(), vd.clone()
    kc[0, L:L + n_q] = ks[0].to(DEV)
    vc[0, L:L + n_q] = vs[0].to(DEV)
    bw = dense_gpu(q, k, v, [L + n_q], causal=True, device_inputs=(q.to(DEV), kc, vc))
    assert np.max(np.abs(a[0] - bw[0])) <= TOL_F32
    assert np.max(np.abs(a[1] - bw[1])) <= 4e-3


def test_step_rows_split_counts(layer_d256):
    """Forced split counts (1, 7, 64) give the same window within tolerance."""
    n_q, L = 3, 2000
    note("step rows split counts")
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, n_q, 16, 256, 1070)
    ks, vs = _steps(1, n_q, 4, 256, 1071)
    ref = steps_ref(q, k, v, [L], ks, vs)
    for S in (1, 7, 64):
        gpu = steps_gpu(q, k, v, [L], ks, vs, num_splits=S, device_inputs=(q.to(DEV), kd, vd))
        assert_close(gpu, ref, what=f"steps S={S}")


def test_step_rows_argument_errors():
    B, n_q, Hq, Hkv, D, cap = 1, 2, 8, 2, 128, 64
    q = torch.zeros((B, n_q, Hq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, cap, Hkv, D), dtype=torch.bfloat16, device=DEV)
    lens = torch.tensor([10], dtype=torch.int32, device=DEV)
    ks = torch.zeros((B, n_q, Hkv, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        ck.decode_attn_steps(q, k, k, lens, ks[:, :1].contiguous(), ks)
    buf = torch.zeros(ks.numel() + 8, dtype=torch.bfloat16, device=DEV)
    odd = buf[1:1 + ks.numel()].view(ks.shape)   # 2-byte aligned only
    with pytest.raises(ck.CkError) as e:
        ck.decode_attn_steps(q, k, k, lens, odd, ks)
    assert e.value.status == -3


# -------------------------------------------------------------- gather ----

@pytest.fixture(scope="module", params=[32768, 65536, 131072])
def sparse_case(request):
    n_kv = request.param
    B, n_q, Hq, Hkv, D = 1, 1, 16, 2, 128
    k, v = synth.kv_cache(B, n_kv, Hkv, D, [n_kv], 1005)
    q = synth.queries(B, n_q, Hq, D, 1005)
    idx = synth.topk_lists(B, n_q, Hkv, n_kv, 2048, 64, seed=5000 + n_kv)
    return n_kv, q, k, v, idx


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gather_matches_oracle(sparse_case, out_dtype):
    n_kv, q, k, v, idx = sparse_case
    note(f"gather n_kv={n_kv} {out_dtype}")
    gpu = gather_gpu(q, k, v, [n_kv], idx, out_dtype=out_dtype)
    assert_close(gpu, oracle_ref(q, k, v, [n_kv], idx=idx), out_dtype, what=f"gather {n_kv}")


def test_masked_scan_matches_oracle_and_gather(sparse_case):
    n_kv, q, k, v, idx = sparse_case
    mask = synth.mask_from_lists(idx, n_kv)
    note(f"masked scan n_kv={n_kv}")
    masked = dense_gpu(q, k, v, [n_kv], keep_mask=mask)
    assert_close(masked, oracle_ref(q, k, v, [n_kv], keep_mask=mask), what=f"masked {n_kv}")
    gathered = gather_gpu(q, k, v, [n_kv], idx)
    assert np.max(np.abs(gathered[0] - masked[0])) <= TOL_F32
    assert np.max(np.abs(gathered[1] - masked[1])) <= 4e-3


@pytest.mark.parametrize("cap,offset", [(1024, 0), (1023, 0), (1024, 1)])
def test_masked_scan_mask_layouts(cap, offset):
    """keep_mask read four cells per load (rows 4-byte aligned) and one per
    load (odd capacity, or a mask pointer off by one byte); any nonzero byte
    keeps its cell.  Causal window, two sequences of different length."""
    B, n_q, Hq, Hkv, D = 2, 3, 8, 2, 128
    lens = [cap - 5, 517]
    note(f"masked scan layout cap={cap} offset={offset}")
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 1021 + cap)
    q = synth.queries(B, n_q, Hq, D, 1022)
    rng = np.random.default_rng(1023 + cap + offset)
    mask = (rng.random((B, n_q, Hkv, cap)) < 0.3) * rng.integers(1, 256, (B, n_q, Hkv, cap))
    mask = mask.astype(np.uint8)
    buf = torch.zeros(mask.size + offset, dtype=torch.uint8, device=DEV)
    mask_d = buf[offset:].view(B, n_q, Hkv, cap)
    mask_d.copy_(torch.from_numpy(mask).to(DEV))
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = ck.decode_attn(q.to(DEV), k.to(DEV), v.to(DEV), lens_d, causal=True, keep_mask=mask_d,
                              return_lse=True)
    torch.cuda.synchronize()
    gpu = (out.cpu().numpy(), lse.cpu().numpy())
    assert_close(gpu, oracle_ref(q, k, v, lens, causal=True, keep_mask=mask), what=f"mask cap={cap}")


def test_gather_lists_edge_entries():
    """Invalid entries (< 0, >= limit, >= capacity), duplicates, shared
    lists, per-query lists under a causal window, ragged list length."""
    B, n_q, Hq, Hkv, D, cap = 2, 3, 8, 2, 128, 700
    lens = np.array([650, 40], dtype=np.int32)
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 77)
    q = synth.queries(B, n_q, Hq, D, 77)
    rng = np.random.default_rng(77)
    W = 101
    idx = rng.integers(-5, cap + 5, size=(B, n_q, Hkv, W), dtype=np.int64).astype(np.int32)
    idx[..., :5] = idx[..., 5:10]        # duplicates
    idx[..., 10] = lens.reshape(B, 1, 1) - 1
    idx[..., 11] = lens.reshape(B, 1, 1)
    for causal in (False, True):
        note(f"gather edge entries causal={causal}")
        gpu = gather_gpu(q, k, v, lens, idx, causal=causal)
        assert_close(gpu, oracle_ref(q, k, v, lens, idx=idx, causal=causal), what="edge lists")
        shared = idx[:, :, 0, :].copy()
        gpu = gather_gpu(q, k, v, lens, shared, causal=causal)
        assert_close(gpu, oracle_ref(q, k, v, lens, idx=shared, causal=causal), what="shared")


# ------------------------------------------------------- exactness checks ----

@pytest.mark.parametrize("cfg", [
    dict(n_q=1, Hq=8, Hkv=2, D=128, cap=1024, lens=[300], causal=False),
    dict(n_q=1, Hq=16, Hkv=4, D=256, cap=24007, lens=[3000], causal=False),
    dict(n_q=4, Hq=16, Hkv=4, D=256, cap=4096, lens=[2000], causal=True),
    dict(n_q=6, Hq=16, Hkv=4, D=256, cap=4096, lens=[4000], causal=True),
    dict(n_q=1, Hq=32, Hkv=8, D=128, cap=32768, lens=[512, 32768, 20000, 777], causal=False),
    dict(n_q=3, Hq=8, Hkv=2, D=128, cap=256, lens=[0, 1, 2, 65, 255], causal=True),
], ids=["tiny", "d256", "window4", "window6", "ragged", "short"])
def test_dense_index_handling_bit_exact(cfg):
    """K = 0 on visible cells (uniform weights) and V[j, d] = bit d of j:
    n * out[d] must round to exactly the number of visible cells with bit d
    set.  NaN fills every cell past the length."""
    note(f"dense bit-exact {cfg}")
    n_q, Hq, Hkv, D, cap, lens, causal = (cfg[x] for x in ("n_q", "Hq", "Hkv", "D", "cap", "lens", "causal"))
    q, k, v = counting_case(n_q, Hq, Hkv, D, cap, lens, 11)
    out, _ = dense_gpu(q, k, v, lens, causal=causal)
    sets = []
    for L in lens:
        per_i = []
        for i in range(n_q):
            lim = max(0, min(L, L - n_q + i + 1)) if causal else L
            per_i.append([np.arange(lim)] * Hkv)
        sets.append(per_i)
    check_counts(out, sets, Hq // Hkv)


@pytest.mark.parametrize("n_kv", [32768, 131072])
def test_gather_and_mask_index_handling_bit_exact(n_kv):
    """The same counting construction through both entries of the sparse
    workload: both recover exactly the listed cell set."""
    Hq, Hkv, D = 16, 2, 128
    q, k, v = counting_case(1, Hq, Hkv, D, n_kv, [n_kv], 12)
    idx = synth.topk_lists(1, 1, Hkv, n_kv, 2048, 64, seed=5000 + n_kv)
    mask = synth.mask_from_lists(idx, n_kv)
    note(f"gather/mask bit-exact n_kv={n_kv}")
    og, _ = gather_gpu(q, k, v, [n_kv], idx)
    om, _ = dense_gpu(q, k, v, [n_kv], keep_mask=mask)
    sets = [[[idx[0, 0, g] for g in range(Hkv)]]]
    check_counts(og, sets, Hq // Hkv)
    check_counts(om, sets, Hq // Hkv)


def test_garbage_past_length_is_never_read():
    """Two caches with the same prefix and different garbage (NaN/Inf bit
    patterns included) give bit-identical outputs."""
    B, n_q, Hq, Hkv, D, cap = 2, 4, 16, 4, 256, 3000
    lens = [2500, 777]
    q = synth.queries(B, n_q, Hq, D, 21)
    k1, v1 = synth.kv_cache(B, cap, Hkv, D, lens, 21)
    k2, v2 = k1.clone(), v1.clone()
    g = synth.generator(99)
    for b, L in enumerate(lens):
        k2[b, L:] = synth.bf16_garbage((cap - L, Hkv, D), g)
        v2[b, L:] = synth.bf16_garbage((cap - L, Hkv, D), g)
    note("garbage invariance")
    a = dense_gpu(q, k1, v1, lens, causal=True)
    b_ = dense_gpu(q, k2, v2, lens, causal=True)
    assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1])
    assert_close(a, oracle_ref(q, k1, v1, lens, causal=True), what="garbage")


@pytest.mark.parametrize("num_splits", [1, 2, 7, 0, 256])
def test_split_count_does_not_change_result(layer_d256, num_splits):
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, 3, 16, 256, 31)
    note(f"split invariance S={num_splits}")
    gpu = dense_gpu(q, k, v, [3000], causal=True, num_splits=num_splits,
                    device_inputs=(q.to(DEV), kd, vd))
    assert_close(gpu, oracle_ref(q, k, v, [3000], causal=True), what=f"S={num_splits}")


def merge_slots(plan, R, D, L, num_splits):
    """Splits per merging lane, rounded up to the kernel's 4, 8 or 16 slots,
    for one sequence of length L under `plan` (the split count, chunk and
    output-group arithmetic the kernel's split merge uses)."""
    tt, target = plan["granule"], num_splits if num_splits else plan["split_target"]
    c = -(-L // target)
    c = max(-(-c // tt) * tt, plan["chunk_min"])
    n_active = -(-L // c)
    nrows = min(R, plan["rows_per_group"])
    ns = 1 if n_active * nrows * D * 4 <= 32 * 1024 else min(plan["slices"], n_active)
    P = nrows * ((D // 4) // ns)
    tpp = 1
    while tpp < 64 and 2 * tpp * P <= 256:
        tpp *= 2
    while tpp < 64 and tpp * 16 < n_active:
        tpp *= 2
    nslot = -(-n_active // tpp)
    return n_active, 4 if nslot <= 4 else 8 if nslot <= 8 else 16


@pytest.mark.parametrize("D,Hq,Hkv,n_q,L,num_splits,slots", [
    (256, 16, 4, 1, 3000, 64, 4),
    (256, 16, 4, 2, 3000, 64, 8),
    (256, 16, 4, 4, 3000, 64, 16),
    (128, 8, 2, 1, 8000, 128, 4),
    (128, 8, 2, 2, 8000, 128, 8),
    (128, 8, 2, 4, 8000, 128, 16),
], ids=lambda x: str(x))
def test_merge_slot_counts(D, Hq, Hkv, n_q, L, num_splits, slots):
    """Each of the merge's slot counts (4, 8 and 16 splits per lane) at both
    head dims, against the oracle: many splits over a causal window, so the
    merging lanes hold full, partial and empty slots."""
    cap = L + 64
    R = n_q * (Hq // Hkv)
    plan = ck.plan(ck.Shape(1, n_q, Hq, Hkv, D, cap), num_splits=num_splits, num_cus=256)
    n_active, got = merge_slots(plan, R, D, L, num_splits)
    assert got == slots and n_active > 1, (n_active, got)
    k, v = synth.kv_cache(1, cap, Hkv, D, [L], 1200 + D + n_q)
    q = synth.queries(1, n_q, Hq, D, 1200 + D + n_q)
    note(f"merge slots {slots}: D={D} n_q={n_q} L={L} S={num_splits} active={n_active}")
    gpu = dense_gpu(q, k, v, [L], causal=n_q > 1, num_splits=num_splits)
    assert_close(gpu, oracle_ref(q, k, v, [L], causal=n_q > 1), what=f"slots {slots}")


@pytest.mark.parametrize("D", [128, 256])
def test_short_span_single_split_threshold(D):
    """Lengths around the automatic single-split threshold (128 KiB of K+V per
    unit: 256 positions at head_dim 128, 128 at 256), plain and as a causal
    window, and a merge small enough to run as one column slice."""
    Hq, Hkv = 8, 2
    edge = 128 * 1024 // (4 * D)
    lens = np.array([edge - 2, edge - 1, edge, edge + 1, edge + 17, 3 * edge], dtype=np.int32)
    cap = int(lens.max()) + 8
    B = len(lens)
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 61 + D)
    for n_q in (1, 3):
        q = synth.queries(B, n_q, Hq, D, 62 + D + n_q)
        note(f"single-split threshold D={D} n_q={n_q} lens={lens.tolist()}")
        gpu = dense_gpu(q, k, v, lens, causal=n_q > 1)
        assert_close(gpu, oracle_ref(q, k, v, lens, causal=n_q > 1), what=f"threshold D={D} n_q={n_q}")


@pytest.mark.parametrize("D", [128, 256])
def test_edge_lengths(D):
    """Empty, single-cell, tile-boundary, full and out-of-range lengths in
    one batch, with a causal window longer than some sequences."""
    cap = 300
    lens = np.array([0, 1, 2, 31, 32, 33, 63, 64, 65, 299, 300, 305, -3], dtype=np.int32)
    B, n_q, Hq, Hkv = len(lens), 3, 8, 2
    k, v = synth.kv_cache(B, cap, Hkv, D, np.clip(lens, 0, cap), 41)
    q = synth.queries(B, n_q, Hq, D, 41)
    for causal in (False, True):
        for num_splits in (0, 1, 3):
            note(f"edge lengths D={D} causal={causal} S={num_splits}")
            gpu = dense_gpu(q, k, v, lens, causal=causal, num_splits=num_splits)
            assert_close(gpu, oracle_ref(q, k, v, lens, causal=causal), what="edges")


@pytest.mark.parametrize("Hq,Hkv,n_q", [(8, 8, 1), (4, 1, 6), (32, 2, 3), (64, 4, 2)])
def test_group_shapes(Hq, Hkv, n_q):
    """Group sizes 1 to 16 and packed row counts from 1 up to 48 (two row
    groups)."""
    D, cap = 128, 900
    lens = [850, 333]
    k, v = synth.kv_cache(2, cap, Hkv, D, lens, 51)
    q = synth.queries(2, n_q, Hq, D, 51)
    note(f"group shapes Hq={Hq} Hkv={Hkv} n_q={n_q}")
    gpu = dense_gpu(q, k, v, lens, causal=True)
    assert_close(gpu, oracle_ref(q, k, v, lens, causal=True), what="groups")


@pytest.mark.parametrize("B,Hq,Hkv,n_q,D,num_splits,rpg,rg", [
    (1, 16, 4, 6, 256, 0, 16, 2),   # two 16-row groups per head, blocks paired on an XCD
    (1, 16, 4, 5, 256, 7, 16, 2),   # 28 (head, split) pairs: the grid's last chunk is padded
    (1, 24, 3, 3, 128, 0, 16, 2),   # three heads: 21 splits, 63 pairs
    (1, 32, 4, 6, 128, 5, 16, 3),   # three groups of 16, 20 pairs padded to 24
    (8, 16, 4, 6, 256, 0, 32, 1),   # batch of 8: 24 rows in one group, two row tiles
    (4, 16, 4, 5, 128, 0, 32, 1),   # batch of 4: 20 rows in one group
    (8, 32, 4, 6, 128, 0, 16, 3),   # 48 rows: 16-row groups at any batch, 2 splits
])
def test_row_group_layouts(B, Hq, Hkv, n_q, D, num_splits, rpg, rg):
    """More than 16 packed rows: 16-row groups sharing tiles (one XCD,
    padded grid) for few heads or more than 32 rows, one 32-row group for
    17-32 rows on many heads; both against the oracle."""
    cap = 2600
    lens = [2500 - 297 * b for b in range(B)]
    p = ck.plan(ck.Shape(B, n_q, Hq, Hkv, D, cap), num_splits=num_splits)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert p["rows_per_group"] == rpg and p["row_groups"] == rg
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 71)
    q = synth.queries(B, n_q, Hq, D, 71)
    note(f"row groups B={B} Hq={Hq} Hkv={Hkv} n_q={n_q} D={D} S={num_splits}")
    gpu = dense_gpu(q, k, v, lens, causal=True, num_splits=num_splits)
    assert_close(gpu, oracle_ref(q, k, v, lens, causal=True), what="row groups")


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_row_groups_edge_lengths(num_splits):
    """Three 16-row groups sharing tiles (48 rows) over empty, one-cell,
    tile-boundary and ragged sequences, with one split (no merge, padded
    grid) or several."""
    B, n_q, Hq, Hkv, D, cap = 5, 6, 16, 2, 128, 300
    lens = np.array([0, 1, 32, 65, 299], dtype=np.int32)
    p = ck.plan(ck.Shape(B, n_q, Hq, Hkv, D, cap), num_splits=num_splits)
    assert p["rows_per_group"] == 16 and p["row_groups"] == 3
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, 74)
    q = synth.queries(B, n_q, Hq, D, 74)
    note(f"row groups edge lengths S={num_splits}")
    gpu = dense_gpu(q, k, v, lens, causal=True, num_splits=num_splits)
    assert_close(gpu, oracle_ref(q, k, v, lens, causal=True), what="row group edges")


@pytest.mark.parametrize("n_q,Hq,Hkv,num_splits", [(2, 32, 1, 0), (2, 32, 1, 3), (3, 128, 4, 0)])
def test_gather_wide_group(n_q, Hq, Hkv, num_splits):
    """32 query heads per KV head: two 16-row groups share the gathered rows
    (2 units of lists), or one 32-row group (12 units of lists)."""
    B, D, n_kv = 1, 128, 20000
    k, v = synth.kv_cache(B, n_kv, Hkv, D, [n_kv], 72)
    q = synth.queries(B, n_q, Hq, D, 72)
    idx = synth.topk_lists(B, n_q, Hkv, n_kv, 2048, 64, seed=73)
    p = ck.plan(ck.Shape(B, n_q, Hq, Hkv, D, n_kv), W=idx.shape[-1], num_splits=num_splits)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert p["rows_per_group"] == (32 if Hkv == 4 else 16)
    note(f"gather G=32 n_q={n_q} Hkv={Hkv} S={num_splits}")
    gpu = gather_gpu(q, k, v, [n_kv], idx, causal=True, num_splits=num_splits)
    assert_close(gpu, oracle_ref(q, k, v, [n_kv], causal=True, idx=idx), what="gather G=32")


def test_head_permutation_within_group(layer_d256):
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, 2, 16, 256, 61)
    perm = torch.tensor([1, 3, 0, 2, 7, 6, 5, 4, 8, 9, 10, 11, 15, 12, 13, 14])
    note("head permutation")
    a, _ = dense_gpu(q, k, v, [5000], causal=True, device_inputs=(q.to(DEV), kd, vd))
    qp = q[:, :, perm].contiguous()
    b, _ = dense_gpu(qp, k, v, [5000], causal=True, device_inputs=(qp.to(DEV), kd, vd))
    assert np.max(np.abs(b - a[:, :, perm.numpy()])) <= 1e-6


# ------------------------------------------------------------ boundary ----

def test_workspace_errors_on_device():
    B, n_q, Hq, Hkv, D, cap = 1, 1, 16, 4, 256, 24007
    q = torch.zeros((B, n_q, Hq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, cap, Hkv, D), dtype=torch.bfloat16, device=DEV)
    lens = torch.full((B,), 5000, dtype=torch.int32, device=DEV)
    need = ck.workspace_size(ck.shape_of(q, k))
    assert need > 0
    small = torch.zeros(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(ck.CkError) as e:
        ck.decode_attn(q, k, k, lens, workspace=small)
    assert e.value.status == -4
    ws = torch.zeros(need + 512, dtype=torch.uint8, device=DEV)
    with pytest.raises(ck.CkError) as e:
        ck.decode_attn(q, k, k, lens, workspace=ws[16:])
    assert e.value.status == -3
    out = ck.decode_attn(q, k, k, lens, workspace=ws[256:])
    torch.cuda.synchronize()
    assert torch.all(out == 0)


def test_released_workspaces_are_rebuilt():
    """Calls after release_workspaces get fresh zeroed workspaces and the
    same results as before (the counters of the old ones are not reused)."""
    note("release workspaces")
    q = synth.queries(1, 1, 16, 256, 1002)
    k, v = synth.kv_cache(1, 3000, 4, 256, [2500], 1002)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lens = torch.tensor([2500], dtype=torch.int32, device=DEV)
    sc = synth.index_scores(1, 1, 4, 3000, 1002).to(DEV)
    a = ck.decode_attn(qd, kd, vd, lens, return_lse=True)
    la = ck.decode_topk(sc, lens, 256, tail=8)
    torch.cuda.synchronize()
    ck.release_workspaces()
    b = ck.decode_attn(qd, kd, vd, lens, return_lse=True)
    lb = ck.decode_topk(sc, lens, 256, tail=8)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(la, lb)
    assert_close((b[0].cpu().numpy(), b[1].cpu().numpy()), oracle_ref(q, k, v, [2500]), what="after release")
