"""GPU: phase timestamps (ck_set_phase_stamps) leave the results bit for bit
as they are, the recorded phases are in order in every workgroup, and the
merge roles account for every column slice once."""

import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
from decode_attention_flash_amd import synth
from gpu_common import DEV, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,L", [(256, 0), (256, 40), (256, 3000), (256, 24000), (128, 300), (128, 5000)])
def test_stamps_change_nothing_and_are_ordered(D, L):
    B, Hq, Hkv, cap = 1, 16 if D == 256 else 8, 4 if D == 256 else 2, 24007
    k, v = synth.kv_cache(B, cap, Hkv, D, [min(L, cap)], 1101, device=DEV)
    q = synth.queries(B, 1, Hq, D, 1101, device=DEV)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    note(f"phase stamps D={D} L={L}")
    ref, ref_lse = ck.decode_attn(q, k, v, lens, return_lse=True)
    pl = ck.plan(ck.shape_of(q, k))
    grid = pl["units"] * pl["splits"]
    stamps = torch.zeros((grid, 16), dtype=torch.int64, device=DEV)
    ck.set_phase_stamps(stamps)
    try:
        out, lse = ck.decode_attn(q, k, v, lens, return_lse=True)
    finally:
        ck.set_phase_stamps(None)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
    t = stamps.cpu().numpy()
    assert np.all(t[:, 0] > 0) and np.all(t[:, 1] >= t[:, 0])  # every workgroup started
    meta = t[:, 15]
    s, n_active, role = meta & 0xFFFF, (meta >> 32) & 0xFFFF, (meta >> 48) & 0xFF
    assert np.all(n_active == n_active[0]) and n_active[0] >= 1
    act = s < n_active
    assert np.sum(act) == n_active[0] * pl["units"]
    a = t[act]
    for k_ in (2, 3, 4, 5):
        ok = a[:, k_] > 0  # a split with no tile (L = 0) stages none
        assert np.all(a[ok, k_] >= a[ok, 1])
    assert np.all(np.diff(a[:, 3:6], axis=1) >= 0)
    if n_active[0] > 1:
        assert np.all(a[:, 6] >= a[:, 5])
        assert sorted(a[a[:, 14] == n_active[0] - 1, 15] >> 48 & 0xFF) == [1] * pl["units"]
        m = a[((a[:, 15] >> 48) & 0xFF) <= 2]
        assert np.all(m[:, 7] >= m[:, 6]) and np.all(m[:, 8] >= m[:, 7])
        # every column slice of every unit merged exactly once (a merge of at
        # most 32 KiB of partials is one slice)
        na = int(n_active[0])
        ns = 1 if na * min(pl["rows"], pl["rows_per_group"]) * D * 4 <= 32 * 1024 else min(pl["slices"], na)
        assert int(np.sum(m[:, 13])) == pl["units"] * ns


def test_stamps_on_step_rows_change_nothing():
    """The step-row entry runs the stamping instance too: same bits."""
    B, n_q, Hq, Hkv, D, cap, L = 1, 3, 16, 4, 256, 4096, 2000
    k, v = synth.kv_cache(B, cap, Hkv, D, [L], 1102, device=DEV)
    q = synth.queries(B, n_q, Hq, D, 1102, device=DEV)
    g = synth.generator(1103)
    ks = synth.bf16_normal((B, n_q, Hkv, D), g).to(DEV)
    vs = synth.bf16_normal((B, n_q, Hkv, D), g).to(DEV)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    note("phase stamps on step rows")
    ref = ck.decode_attn_steps(q, k, v, lens, ks, vs)
    pl = ck.plan(ck.shape_of(q, k))
    stamps = torch.zeros((pl["units"] * pl["splits"], 16), dtype=torch.int64, device=DEV)
    ck.set_phase_stamps(stamps)
    try:
        out = ck.decode_attn_steps(q, k, v, lens, ks, vs)
    finally:
        ck.set_phase_stamps(None)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert int((stamps[:, 0] > 0).sum()) == pl["units"] * pl["splits"]  # the stamping instance ran


def active_splits(pl, rows, D, L):
    """Active splits per unit of plain automatic-split decode with one row
    group per head whose units leave most of the 256 CUs idle: three quarters
    of the split target, at most 32 for windows of 8 or more rows at head_dim
    256 up to 6144 positions; the range is cut in whole granules."""
    S = max(1, pl["split_target"] * 3 // 4)
    if rows >= 8 and D == 256 and L <= 6144:
        S = min(S, 32)
    gran = pl["granule"]
    c = max(-(-(-(-L // S)) // gran) * gran, pl["chunk_min"])
    need = -(-(-(-L // pl["splits"])) // gran) * gran
    return -(-L // max(c, need))


@pytest.mark.parametrize("n_q,L", [(1, 4000), (2, 3000), (3, 4000), (3, 6144), (3, 6145), (4, 6000), (4, 8000)])
def test_window_split_count(n_q, L):
    """The active split count the kernel takes for causal windows, read from
    the stamps, on both sides of the 6144-position window bound; the stamped
    launch gives the plain launch's bits."""
    B, Hq, Hkv, D, cap = 1, 16, 4, 256, 8192
    k, v = synth.kv_cache(B, cap, Hkv, D, [L], 1104 + n_q, device=DEV)
    q = synth.queries(B, n_q, Hq, D, 1104 + n_q, device=DEV)
    lens = torch.tensor([L], dtype=torch.int32, device=DEV)
    note(f"window split count n_q={n_q} L={L}")
    ref = ck.decode_attn(q, k, v, lens, causal=True)
    pl = ck.plan(ck.shape_of(q, k))
    assert pl["units"] == 4 and pl["row_groups"] == 1
    stamps = torch.zeros((pl["units"] * pl["splits"], 16), dtype=torch.int64, device=DEV)
    ck.set_phase_stamps(stamps)
    try:
        out = ck.decode_attn(q, k, v, lens, causal=True)
    finally:
        ck.set_phase_stamps(None)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    n_active = (stamps[:, 15].cpu().numpy() >> 32) & 0xFFFF
    want = active_splits(pl, n_q * (Hq // Hkv), D, L)
    assert np.all(n_active == want), (sorted(set(n_active.tolist())), want)
