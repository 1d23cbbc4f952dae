"""Bounded waits that give up do so visibly (GPU).

A split-merge helper waits for the unit's last split, and top-k row
workgroups wait at barriers.  Neither wait can fail while the launch's
workgroups all run, so the failure is forced from the host: the test
presets a workspace counter so that the awaited arrival can never happen
(an arrival count that starts at -1 never reaches the split count; a row
barrier count that starts at -P never reaches P) and lowers the poll limit
so the give-up comes in a millisecond.  Every kernel must still end
normally (the synchronize returns, nothing faults), the workspace status
word must name the give-up, the merge's slices must read NaN, and after the
limit is restored and the workspace zeroed the same buffer must give the
oracle's result again."""
import math

import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
import oracle
from decode_attention_flash_amd import synth
from gpu_common import DEV, assert_close, counters_ready, note, oracle_ref

pytestmark = pytest.mark.gpu


def test_merge_helper_gives_up_visibly():
    B, n_q, Hq, Hkv, D, cap, L = 1, 1, 16, 4, 256, 8192, 8000
    k, v = synth.kv_cache(B, cap, Hkv, D, [L], 1002)
    q = synth.queries(B, n_q, Hq, D, 1002)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    shape = ck.shape_of(qd, kd)
    assert ck.plan(shape)["slices"] > 1
    ws = ck.new_workspace(shape)
    units = ck.plan(shape)["units"]
    # unit u's counters: 512 ints after the 256-byte header; parity 0 names
    # the set at ints 128.., whose arrival count is at +32
    w = ws.view(torch.int32)
    for u in range(units):
        w[64 + 512 * u + 128 + 32] = -1
    note("merge give-up: arrivals start at -1, poll limit 1000")
    ck.set_spin_limit(1000)
    try:
        out = ck.decode_attn(qd, kd, vd, lens, workspace=ws)
        torch.cuda.synchronize()
        status = ck.workspace_status(ws)
    finally:
        ck.set_spin_limit(0)
    assert status == ck.CK_WS_ERR_MERGE
    o = out.cpu().numpy()
    assert np.isnan(o).any()  # the helpers' slices
    # zero the workspace and run again: the oracle's result, status 0
    ws.zero_()
    out, lse = ck.decode_attn(qd, kd, vd, lens, workspace=ws, return_lse=True)
    torch.cuda.synchronize()
    assert ck.workspace_status(ws) == 0
    assert counters_ready(ws, units)
    assert_close((out.cpu().numpy(), lse.cpu().numpy()), oracle_ref(q, k, v, [L]), what="after give-up")


def test_topk_barrier_gives_up_visibly():
    B, n_q, Hs, cap, L, kk, tail = 1, 1, 2, 131072, 131072, 2048, 64
    sc = synth.index_scores(B, n_q, Hs, cap, 1005)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    scd = sc.to(DEV)
    p = ck.topk_plan((B, n_q, Hs, cap), kk, tail)
    assert p["wgs_per_row"] > 1 and p["workspace_bytes"] > 0
    ws = torch.zeros(p["workspace_bytes"], dtype=torch.uint8, device=DEV)
    P = p["wgs_per_row"]
    # row 0's barrier count of counter set 0 (the set a zeroed workspace's
    # parity names): word 16 of the row, after the 256-byte header
    ws.view(torch.int32)[64 + 16] = -P
    note("top-k give-up: row barrier count starts at -P, poll limit 1000")
    ck.set_spin_limit(1000)
    try:
        ck.decode_topk(scd, lens, kk, tail=tail, workspace=ws)
        torch.cuda.synchronize()
        status = ck.workspace_status(ws)
    finally:
        ck.set_spin_limit(0)
    assert status == ck.CK_WS_ERR_TOPK
    ws.zero_()
    got = ck.decode_topk(scd, lens, kk, tail=tail, workspace=ws)
    torch.cuda.synchronize()
    assert ck.workspace_status(ws) == 0
    ref = oracle.topk(sc.numpy(), np.array([L], np.int32), kk, tail)
    assert np.array_equal(got.cpu().numpy(), ref)
