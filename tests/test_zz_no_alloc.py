"""ck_decode_attn_noalloc against ck_decode_attn (GPU).

The no-allocation entry point runs the same kernels as ck_decode_attn with
the split merge's workspace in the library's file-scope per-device scratch.
Two calls in a row, the second on a smaller input (and a different plan),
must each give ck_decode_attn's result bit for bit (the same kernel and
plan: only where the partials live differs) and the oracle's within the
stated tolerance; a third call on the first shape checks that the scratch
left by a different shape serves it again.  A shape whose plan does not fit
the scratch is refused before any launch."""
import math

import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
from decode_attention_flash_amd import synth
from gpu_common import DEV, assert_close, note, oracle_ref

pytestmark = pytest.mark.gpu


def run_both(B, n_q, Hq, Hkv, D, cap, lens, seed, causal=False):
    k, v = synth.kv_cache(B, cap, Hkv, D, lens, seed)
    q = synth.queries(B, n_q, Hq, D, seed)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lens_d = torch.as_tensor(lens, dtype=torch.int32).to(DEV)
    note(f"no-alloc B={B} n_q={n_q} Hq={Hq} Hkv={Hkv} D={D} cap={cap} lens={lens[:4]}")
    a, la = ck.decode_attn_noalloc(qd, kd, vd, lens_d, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    b, lb = ck.decode_attn(qd, kd, vd, lens_d, causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert_close((a.cpu().numpy(), la.cpu().numpy()), oracle_ref(q, k, v, lens, causal=causal), what="no-alloc")


def test_noalloc_matches_decode_attn_two_calls():
    # a long head_dim-256 layer (64 splits per head), then a smaller batch of
    # short causal windows at head_dim 128 (other units, other splits)
    run_both(1, 1, 16, 4, 256, 12000, [11000], 2001)
    run_both(2, 3, 8, 2, 128, 3000, [2500, 700], 2002, causal=True)
    run_both(1, 1, 16, 4, 256, 12000, [6000], 2003)


def test_noalloc_refuses_plans_past_the_scratch():
    # 64 sequences x 32 KV heads = 2048 units: more counters than the scratch holds
    B, Hq, Hkv, D, cap = 64, 32, 32, 128, 256
    q = torch.zeros((B, 1, Hq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, cap, Hkv, D), dtype=torch.bfloat16, device=DEV)
    lens = torch.full((B,), cap, dtype=torch.int32, device=DEV)
    p = ck.plan(ck.shape_of(q, k), num_splits=2)
    assert p["splits"] == 2 and p["units"] == 2048
    with pytest.raises(ck.CkError) as e:
        ck.decode_attn_noalloc(q, k, k, lens, num_splits=2)
    assert e.value.status == -6
