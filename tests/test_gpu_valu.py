"""GPU parity of the VALU contractions (ck_set_contraction): dense and
gathered decode of up to 8 packed rows with QK^T and PV on v_dot2 over bf16
pairs (CK_CONTRACT_VALU) or in plain fp32 (CK_CONTRACT_VALU_F32) instead of
MFMA, against the fp64 oracle to the same tolerances, with the same
bit-exact index handling, and against the MFMA kernel on the same inputs."""

import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
from decode_attention_flash_amd import synth
from gpu_common import (DEV, TOL_F32, assert_close, check_counts, counting_case, dense_gpu, gather_gpu, note,
                        oracle_ref)

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["valu", "valu_f32"])
def valu(request):
    ck.set_contraction(request.param)
    try:
        yield request.param
    finally:
        ck.set_contraction("mfma")


@pytest.fixture(scope="module")
def layer_d256():
    B, Hq, Hkv, D, cap = 1, 16, 4, 256, 24007
    k, v = synth.kv_cache(B, cap, Hkv, D, [24000], 1002)
    return k, v, (k.to(DEV), v.to(DEV))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiny_dense(valu, out_dtype):
    """B=1, Hq=8, Hkv=2, D=128, capacity 1024, 300 filled: 4 rows."""
    note(f"valu tiny dense {out_dtype}")
    k, v = synth.kv_cache(1, 1024, 2, 128, [300], 1001)
    q = synth.queries(1, 1, 8, 128, 1001)
    assert_close(dense_gpu(q, k, v, [300], out_dtype=out_dtype), oracle_ref(q, k, v, [300]), out_dtype,
                 "valu tiny")


@pytest.mark.parametrize("L", [1000, 8000, 24000])
def test_d256_plain_decode(layer_d256, valu, L):
    note(f"valu D=256 L={L}")
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, 1, 16, 256, 1002)
    gpu = dense_gpu(q, k, v, [L], device_inputs=(q.to(DEV), kd, vd))
    assert_close(gpu, oracle_ref(q, k, v, [L]), what=f"valu L={L}")


def test_d256_two_query_causal_window(layer_d256, valu):
    """n_q = 2 with a group of 4: 8 rows, each with its own causal limit."""
    note("valu D=256 n_q=2 causal")
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, 2, 16, 256, 1033)
    gpu = dense_gpu(q, k, v, [4000], causal=True, device_inputs=(q.to(DEV), kd, vd))
    assert_close(gpu, oracle_ref(q, k, v, [4000], causal=True), what="valu n_q=2")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gather(valu, out_dtype):
    """Hq=16, Hkv=2 (8 rows per head), 2048 listed cells plus the last 64."""
    n_kv = 32768
    k, v = synth.kv_cache(1, n_kv, 2, 128, [n_kv], 1005)
    q = synth.queries(1, 1, 16, 128, 1005)
    idx = synth.topk_lists(1, 1, 2, n_kv, 2048, 64, seed=5000 + n_kv)
    note(f"valu gather {out_dtype}")
    gpu = gather_gpu(q, k, v, [n_kv], idx, out_dtype=out_dtype)
    assert_close(gpu, oracle_ref(q, k, v, [n_kv], idx=idx), out_dtype, "valu gather")


def test_gather_causal_queries(valu):
    """Three queries with causal limits over their own lists (8 rows each):
    the limit cuts the tail of the later lists differently per query."""
    n_kv, L = 8192, 8000
    k, v = synth.kv_cache(2, n_kv, 2, 128, [L, 5000], 1006)
    q = synth.queries(2, 3, 16, 128, 1006)
    idx = synth.topk_lists(2, 3, 2, n_kv, 512, 64, seed=5123)
    note("valu gather causal n_q=3")
    gpu = gather_gpu(q, k, v, [L, 5000], idx, causal=True)
    assert_close(gpu, oracle_ref(q, k, v, [L, 5000], causal=True, idx=idx), what="valu gather causal")


def test_batched_ragged(valu):
    """B=32, Hq=32, Hkv=8, D=128, capacity 32768, lengths uniform in
    [512, 32768]: every sequence against the oracle."""
    B, Hq, Hkv, D, cap = 32, 32, 8, 128, 32768
    note("valu batched ragged")
    k, v = synth.kv_cache(B, cap, Hkv, D, [cap] * B, 1004, device=DEV, garbage=False)
    q = synth.queries(B, 1, Hq, D, 1004, device=DEV)
    lens = synth.ragged_lens(B, 512, cap, 4100)
    lens_d = torch.from_numpy(lens).to(DEV)
    o, l = ck.decode_attn(q, k, v, lens_d, return_lse=True)
    torch.cuda.synchronize()
    assert_close((o.cpu().numpy(), l.cpu().numpy()), oracle_ref(q.cpu(), k.cpu(), v.cpu(), lens),
                 what="valu ragged")


@pytest.mark.parametrize("D", [128, 256])
def test_edge_lengths(valu, D):
    """Empty, single-cell, tile-boundary, full and out-of-range lengths, one
    and two queries (4 and 8 rows), split counts 0, 1 and 3."""
    cap = 300
    lens = np.array([0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 299, 300, 305, -3], dtype=np.int32)
    B, Hq, Hkv = len(lens), 8, 2
    k, v = synth.kv_cache(B, cap, Hkv, D, np.clip(lens, 0, cap), 41)
    for n_q in (1, 2):
        q = synth.queries(B, n_q, Hq, D, 41 + n_q)
        for causal in (False, True):
            for num_splits in (0, 1, 3):
                note(f"valu edge lengths D={D} n_q={n_q} causal={causal} S={num_splits}")
                gpu = dense_gpu(q, k, v, lens, causal=causal, num_splits=num_splits)
                assert_close(gpu, oracle_ref(q, k, v, lens, causal=causal), what="valu edges")


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 128), (6, 3, 256), (12, 4, 128), (10, 2, 256), (24, 3, 128)])
def test_group_sizes(valu, Hq, Hkv, D):
    """Groups of 1, 2, 3, 5 and 8 rows (padding rows inside the 4- and 8-row
    lane layouts)."""
    cap, lens = 900, [850, 333]
    k, v = synth.kv_cache(2, cap, Hkv, D, lens, 51)
    q = synth.queries(2, 1, Hq, D, 51)
    note(f"valu groups Hq={Hq} Hkv={Hkv} D={D}")
    assert_close(dense_gpu(q, k, v, lens), oracle_ref(q, k, v, lens), what="valu groups")


@pytest.mark.parametrize("cfg", [
    dict(n_q=1, Hq=8, Hkv=2, D=128, cap=1024, lens=[300]),
    dict(n_q=1, Hq=16, Hkv=4, D=256, cap=24007, lens=[3000]),
    dict(n_q=2, Hq=8, Hkv=2, D=256, cap=256, lens=[0, 1, 2, 65, 255]),
], ids=["tiny", "d256", "short"])
def test_dense_index_handling_bit_exact(valu, cfg):
    """K = 0 on visible cells and V[j, d] = bit d of j (NaN past the length):
    n * out[d] rounds to exactly the count of visible cells with bit d set."""
    note(f"valu dense bit-exact {cfg}")
    n_q, Hq, Hkv, D, cap, lens = (cfg[x] for x in ("n_q", "Hq", "Hkv", "D", "cap", "lens"))
    causal = n_q > 1
    q, k, v = counting_case(n_q, Hq, Hkv, D, cap, lens, 11)
    out, _ = dense_gpu(q, k, v, lens, causal=causal)
    sets = [[[np.arange(max(0, min(L, L - n_q + i + 1)) if causal else L)] * Hkv for i in range(n_q)]
            for L in lens]
    check_counts(out, sets, Hq // Hkv)


def test_gather_index_handling_bit_exact(valu):
    n_kv, Hq, Hkv, D = 32768, 16, 2, 128
    q, k, v = counting_case(1, Hq, Hkv, D, n_kv, [n_kv], 12)
    idx = synth.topk_lists(1, 1, Hkv, n_kv, 2048, 64, seed=5000 + n_kv)
    note("valu gather bit-exact")
    og, _ = gather_gpu(q, k, v, [n_kv], idx)
    check_counts(og, [[[idx[0, 0, g] for g in range(Hkv)]]], Hq // Hkv)


@pytest.mark.parametrize("kind", ["valu", "valu_f32"])
def test_agrees_with_mfma(layer_d256, kind):
    """Same inputs through MFMA and a VALU contraction: equal within the fp32
    tolerance (the dot2 form rounds the probabilities to bf16 as MFMA does and
    differs only in the order of fp32 sums; the fp32 form keeps them in fp32),
    and not bit-identical, which shows that the second launch took the other
    kernel."""
    k, v, (kd, vd) = layer_d256
    q = synth.queries(1, 1, 16, 256, 1077)
    note(f"{kind} vs mfma D=256 L=8000")
    ck.set_contraction("mfma")
    a, la = dense_gpu(q, k, v, [8000], device_inputs=(q.to(DEV), kd, vd))
    ck.set_contraction(kind)
    try:
        b, lb = dense_gpu(q, k, v, [8000], device_inputs=(q.to(DEV), kd, vd))
    finally:
        ck.set_contraction("mfma")
    assert float(np.max(np.abs(a - b))) <= TOL_F32
    assert float(np.max(np.abs(la - lb))) <= 4e-3
    assert not np.array_equal(a, b)

