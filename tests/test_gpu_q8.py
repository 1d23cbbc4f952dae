"""GPU parity for the paged INT8 KV cache: the append kernel against the
oracle's quantizer and placement (bit-exact codes and scales), attention
over pages built by the oracle against the oracle, rollback, and a decode
loop replayed from a captured HIP graph."""
import math

import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
import oracle
from decode_attention_flash_amd import synth
from gpu_common import DEV, assert_close, counters_ready, note

pytestmark = pytest.mark.gpu


def host_pages(num_pages, page, Hkv, D):
    kq = np.zeros((num_pages, Hkv, page, D), np.int8)
    ksc = np.zeros((num_pages, Hkv, page), np.float32)
    return kq, kq.copy(), ksc, ksc.copy()


def to_device(cache: ck.PagedQ8Cache, kq, vq, ksc, vsc):
    cache.k_codes.copy_(torch.from_numpy(kq))
    cache.v_codes.copy_(torch.from_numpy(vq))
    cache.k_scales.copy_(torch.from_numpy(ksc))
    cache.v_scales.copy_(torch.from_numpy(vsc))


def tables(B, max_pages, num_pages, seed):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_pages)
    return perm[:B * max_pages].reshape(B, max_pages).astype(np.int32)


def filled_case(B, Hkv, D, page, max_pages, lens, seed, extra_pages=3):
    """A page pool filled by the oracle's append with the first lens[b]
    tokens of each sequence (random N(0,1) rows; other cells zero)."""
    num_pages = B * max_pages + extra_pages
    bt = tables(B, max_pages, num_pages, seed)
    kq, vq, ksc, vsc = host_pages(num_pages, page, Hkv, D)
    n = int(max(lens))
    gen = synth.generator(seed)
    k_all = synth.bf16_normal((B, max(n, 1), Hkv, D), gen)
    v_all = synth.bf16_normal((B, max(n, 1), Hkv, D), gen)
    if n > 0:
        # append sequence by sequence so each gets exactly lens[b] rows
        for b in range(B):
            if lens[b] == 0:
                continue
            one = np.zeros(B, np.int32)
            sel_k = torch.zeros((B, lens[b], Hkv, D), dtype=torch.bfloat16)
            sel_v = torch.zeros_like(sel_k)
            sel_k[b], sel_v[b] = k_all[b, :lens[b]], v_all[b, :lens[b]]
            bt_b = np.full_like(bt, -1)
            bt_b[b] = bt[b]
            oracle.q8_append(sel_k, sel_v, one, bt_b, kq, vq, ksc, vsc)
    return bt, (kq, vq, ksc, vsc), num_pages


def make_cache(bt, pages, num_pages, page, Hkv, D):
    c = ck.PagedQ8Cache(num_pages, page, Hkv, D, torch.from_numpy(bt).to(DEV))
    to_device(c, *pages)
    return c


# ------------------------------------------------------------------ append ----

@pytest.mark.parametrize("D", [128, 256])
def test_append_bit_exact(D):
    """Codes and scales of the append kernel equal the oracle's bit for bit,
    across page boundaries, with rows past the capacity and a page outside
    the pool dropped, and an all-zero row."""
    B, Hkv, page, max_pages, n_new = 3, 2, 64, 3, 70
    num_pages = B * max_pages + 2
    note(f"q8 append D={D}")
    bt = tables(B, max_pages, num_pages, 2000 + D)
    bt[2, 1] = num_pages + 5                      # outside the pool: dropped
    gen = synth.generator(2001 + D)
    k_new = synth.bf16_normal((B, n_new, Hkv, D), gen) * 4
    v_new = synth.bf16_normal((B, n_new, Hkv, D), gen)
    k_new[0, 3] = 0                               # all-zero rows: scale 0
    start = np.array([10, 150, 60], np.int32)     # the second runs past capacity 192
    ref = host_pages(num_pages, page, Hkv, D)
    oracle.q8_append(k_new, v_new, start, bt, *ref)
    c = ck.PagedQ8Cache(num_pages, page, Hkv, D, torch.from_numpy(bt).to(DEV))
    ck.kv_append_q8(c, k_new.to(DEV), v_new.to(DEV), torch.from_numpy(start).to(DEV))
    torch.cuda.synchronize()
    got = (c.k_codes.cpu().numpy(), c.v_codes.cpu().numpy(), c.k_scales.cpu().numpy(), c.v_scales.cpu().numpy())
    for g, r, name in zip(got, ref, ("k codes", "v codes", "k scales", "v scales")):
        assert np.array_equal(g.view(np.uint8) if g.dtype == np.int8 else g.view(np.uint32),
                              r.view(np.uint8) if r.dtype == np.int8 else r.view(np.uint32)), name


# --------------------------------------------------------------- attention ----

@pytest.mark.parametrize("L", [1, 100, 3000, 8000])
def test_d256_decode_matches_oracle(L):
    """Hq=16, Hkv=4, D=256 decode over pages of 128 tokens in a shuffled pool."""
    B, Hq, Hkv, D, page, max_pages = 1, 16, 4, 256, 128, 64
    note(f"q8 D=256 decode L={L}")
    bt, pages, num_pages = filled_case(B, Hkv, D, page, max_pages, [L], 2100 + L)
    c = make_cache(bt, pages, num_pages, page, Hkv, D)
    q = synth.queries(B, 1, Hq, D, 2101)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    out, lse = ck.decode_attn_q8(q.to(DEV), c, lens, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.attn_q8(q, *pages, bt, np.array([L], np.int32), 1 / math.sqrt(D))
    assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what=f"q8 L={L}")


@pytest.mark.parametrize("D,L", [(128, 16384), (128, 16447), (128, 20000), (256, 19000)])
def test_long_block_table(D, L):
    """A block table of 320 entries (64-token pages): the first tile of a
    split that starts within the first 256 entries takes its page from the
    entries loaded with the length, a later one from its own load."""
    B, Hkv, page, max_pages = 1, 2, 64, 320
    Hq = 8 if D == 128 else 4
    note(f"q8 long block table D={D} L={L}")
    bt, pages, num_pages = filled_case(B, Hkv, D, page, max_pages, [L], 2150 + L)
    c = make_cache(bt, pages, num_pages, page, Hkv, D)
    q = synth.queries(B, 1, Hq, D, 2151)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    for num_splits in (0, 16):
        out, lse = ck.decode_attn_q8(q.to(DEV), c, lens, return_lse=True, num_splits=num_splits)
        torch.cuda.synchronize()
        ref = oracle.attn_q8(q, *pages, bt, np.array([L], np.int32), 1 / math.sqrt(D))
        assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what=f"q8 long table L={L} S={num_splits}")


@pytest.mark.parametrize("n_q", [3, 4, 6])
@pytest.mark.parametrize("L", [2000, 4000, 6144, 6145])  # 6144: the last span with the window split cap
def test_d256_causal_window_matches_oracle(n_q, L):
    B, Hq, Hkv, D, page, max_pages = 1, 16, 4, 256, 64, 100
    note(f"q8 window n_q={n_q} L={L}")
    bt, pages, num_pages = filled_case(B, Hkv, D, page, max_pages, [L], 2200 + n_q)
    c = make_cache(bt, pages, num_pages, page, Hkv, D)
    q = synth.queries(B, n_q, Hq, D, 2201)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    for out_dtype in (torch.float32, torch.bfloat16):
        out, lse = ck.decode_attn_q8(q.to(DEV), c, lens, causal=True, out_dtype=out_dtype, return_lse=True)
        torch.cuda.synchronize()
        ref = oracle.attn_q8(q, *pages, bt, np.array([L], np.int32), 1 / math.sqrt(D), True)
        assert_close((out.float().cpu().numpy(), lse.cpu().numpy()), ref, out_dtype, f"q8 window {n_q} L={L}")


@pytest.mark.parametrize("B,Hq,Hkv,D,lens,rpg", [
    (4, 16, 4, 256, [2000, 1234, 0, 2500], 32),  # 24 rows on 16 pairs: one 32-row group
    (1, 32, 4, 128, [2500], 16),                 # 48 rows: three 16-row groups sharing tiles
])
def test_window_row_groups(B, Hq, Hkv, D, lens, rpg):
    n_q, page, max_pages = 6, 64, 40
    note(f"q8 window B={B} Hq={Hq} D={D}")
    p = ck.plan(ck.Shape(B, n_q, Hq, Hkv, D, page * max_pages))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert p["rows_per_group"] == rpg
    bt, pages, num_pages = filled_case(B, Hkv, D, page, max_pages, lens, 2300 + B)
    c = make_cache(bt, pages, num_pages, page, Hkv, D)
    q = synth.queries(B, n_q, Hq, D, 2301)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = ck.decode_attn_q8(q.to(DEV), c, lens_d, causal=True, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.attn_q8(q, *pages, bt, np.array(lens, np.int32), 1 / math.sqrt(D), True)
    assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what=f"q8 window B={B}")


def test_d128_ragged_batch_matches_oracle():
    """B=6 ragged lengths (one empty, one at a page boundary), one table entry
    inside a sequence pointing outside the pool (its tokens read as zeros)."""
    B, Hq, Hkv, D, page, max_pages = 6, 32, 8, 128, 64, 40
    lens = [0, 64, 1, 777, 2560, 1999]
    note("q8 D=128 ragged batch")
    bt, pages, num_pages = filled_case(B, Hkv, D, page, max_pages, lens, 2300)
    bt[3, 5] = 10 ** 6
    c = make_cache(bt, pages, num_pages, page, Hkv, D)
    q = synth.queries(B, 1, Hq, D, 2301)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = ck.decode_attn_q8(q.to(DEV), c, lens_d, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.attn_q8(q, *pages, bt, np.array(lens, np.int32), 1 / math.sqrt(D))
    assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what="q8 ragged")


def test_full_size_ragged_batch():
    """The bench's ragged INT8 batch (B=32, Hq=32, Hkv=8, D=128, 128-token
    pages, capacity 32768, lengths U[512, 32768]) in the launch the bench
    times (default plan): every page of the pool holds random codes and
    scales (drawn on the device, copied to the host for the oracle), the
    block table is a random permutation of the pool, and every sequence is
    checked against the oracle."""
    B, Hq, Hkv, D, page, cap = 32, 32, 8, 128, 128, 32768
    max_pages = cap // page
    num_pages = B * max_pages
    lens = synth.ragged_lens(B, 512, cap, 4000)
    bt = tables(B, max_pages, num_pages, 2600)
    c = ck.PagedQ8Cache(num_pages, page, Hkv, D, torch.from_numpy(bt).to(DEV))
    g = torch.Generator(device=DEV)
    g.manual_seed(2601)
    note("q8 full-size ragged batch: filling the pool")
    c.k_codes.copy_(torch.randint(-127, 128, c.k_codes.shape, generator=g, device=DEV, dtype=torch.int8))
    c.v_codes.copy_(torch.randint(-127, 128, c.v_codes.shape, generator=g, device=DEV, dtype=torch.int8))
    c.k_scales.uniform_(0.005, 0.03, generator=g)
    c.v_scales.uniform_(0.005, 0.03, generator=g)
    q = synth.queries(B, 1, Hq, D, 2602)
    note("q8 full-size ragged batch: launch")
    out, lse = ck.decode_attn_q8(q.to(DEV), c, torch.from_numpy(lens).to(DEV), return_lse=True)
    torch.cuda.synchronize()
    pages = [c.k_codes.cpu().numpy(), c.v_codes.cpu().numpy(), c.k_scales.cpu().numpy(), c.v_scales.cpu().numpy()]
    ref = oracle.attn_q8(q, *pages, bt, lens.astype(np.int32), 1 / math.sqrt(D))
    assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what=f"q8 full size (all {B} sequences)")


def test_split_counts_agree():
    B, Hq, Hkv, D, page, max_pages, L = 1, 8, 2, 128, 64, 32, 1500
    note("q8 split counts")
    bt, pages, num_pages = filled_case(B, Hkv, D, page, max_pages, [L], 2400)
    c = make_cache(bt, pages, num_pages, page, Hkv, D)
    q = synth.queries(B, 1, Hq, D, 2401)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    ref = oracle.attn_q8(q, *pages, bt, np.array([L], np.int32), 1 / math.sqrt(D))
    for S in (1, 5, 64):
        out, lse = ck.decode_attn_q8(q.to(DEV), c, lens, num_splits=S, return_lse=True)
        torch.cuda.synchronize()
        assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what=f"q8 S={S}")


# ---------------------------------------------------------------- rollback ----

def test_rollback_then_append():
    """Append 6 draft tokens, accept 2 (lower the length), append 3 more: the
    pages equal the oracle's after the same steps, and attention over the
    final length matches the oracle."""
    B, Hq, Hkv, D, page, max_pages, L0 = 2, 16, 4, 256, 64, 8, 100
    note("q8 rollback")
    bt, pages, num_pages = filled_case(B, Hkv, D, page, max_pages, [L0, L0 + 30], 2500)
    c = make_cache(bt, pages, num_pages, page, Hkv, D)
    gen = synth.generator(2501)
    drafts = (synth.bf16_normal((B, 6, Hkv, D), gen), synth.bf16_normal((B, 6, Hkv, D), gen))
    more = (synth.bf16_normal((B, 3, Hkv, D), gen), synth.bf16_normal((B, 3, Hkv, D), gen))
    lens = np.array([L0, L0 + 30], np.int32)
    lens_d = torch.from_numpy(lens).to(DEV)
    ck.kv_append_q8(c, drafts[0].to(DEV), drafts[1].to(DEV), lens_d)
    oracle.q8_append(drafts[0], drafts[1], lens, bt, *pages)
    lens = lens + 2                     # two drafts accepted, four rolled back
    lens_d.copy_(torch.from_numpy(lens))
    ck.kv_append_q8(c, more[0].to(DEV), more[1].to(DEV), lens_d)
    oracle.q8_append(more[0], more[1], lens, bt, *pages)
    lens = lens + 3
    lens_d.copy_(torch.from_numpy(lens))
    torch.cuda.synchronize()
    assert np.array_equal(c.k_codes.cpu().numpy(), pages[0]) and np.array_equal(c.v_codes.cpu().numpy(), pages[1])
    assert np.array_equal(c.k_scales.cpu().numpy(), pages[2]) and np.array_equal(c.v_scales.cpu().numpy(), pages[3])
    q = synth.queries(B, 1, Hq, D, 2502)
    out, lse = ck.decode_attn_q8(q.to(DEV), c, lens_d, return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.attn_q8(q, *pages, bt, lens, 1 / math.sqrt(D))
    assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what="q8 rollback")


def test_decode_loop_graph_replay():
    """One captured decode step (append the new token, advance the length,
    attend) replayed 4 times with new token values in place: every step
    matches the oracle run on the same steps."""
    B, Hq, Hkv, D, page, max_pages = 2, 16, 4, 256, 64, 8
    L0 = [63, 200]
    note("q8 decode loop graph")
    bt, pages, num_pages = filled_case(B, Hkv, D, page, max_pages, L0, 2600)
    c = make_cache(bt, pages, num_pages, page, Hkv, D)
    lens = np.array(L0, np.int32)
    lens_d = torch.from_numpy(lens).to(DEV)
    k_new = torch.zeros((B, 1, Hkv, D), dtype=torch.bfloat16, device=DEV)
    v_new = torch.zeros_like(k_new)
    q_d = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, Hq), dtype=torch.float32, device=DEV)
    shape = ck.Shape(B, 1, Hq, Hkv, D, c.capacity)
    ws = ck.new_workspace(shape)

    def step():
        ck.kv_append_q8(c, k_new, v_new, lens_d)
        lens_d.add_(1)
        ck.decode_attn_q8(q_d, c, lens_d, out=out, lse=lse, workspace=ws)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        step()
    torch.cuda.synchronize()
    gen = synth.generator(2601)
    for r in range(4):
        kn, vn = synth.bf16_normal((B, 1, Hkv, D), gen), synth.bf16_normal((B, 1, Hkv, D), gen)
        q = synth.queries(B, 1, Hq, D, 2610 + r)
        k_new.copy_(kn.to(DEV))
        v_new.copy_(vn.to(DEV))
        q_d.copy_(q.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        oracle.q8_append(kn, vn, lens, bt, *pages)
        lens = lens + 1
        assert np.array_equal(lens_d.cpu().numpy(), lens)
        ref = oracle.attn_q8(q, *pages, bt, lens, 1 / math.sqrt(D))
        assert_close((out.cpu().numpy(), lse.cpu().numpy()), ref, what=f"q8 loop step {r}")
    assert counters_ready(ws, ck.plan(shape)["units"])
