"""Stress of the in-launch split merge (GPU).

The merge's arrival counting, slice claims and counter reset run once per
launch; a race among them would show as a wrong result on an occasional
launch.  Each case captures one launch in a graph and replays it 1000 times
with fresh lengths written into the device length buffer before each
replay, for the automatic plan and for forced split counts 2, 7 and 64.
After every replay an eager launch on the same lengths (its own output
buffers, the same workspace) must give the same bits (also for causal windows,
whose split count changes at 6144 positions); the case stops at
the first mismatch.  At the end the workspace's status word is zero and
its counters are ready for the next launch."""
import numpy as np
import pytest
import torch

import decode_attention_flash_amd as ck
from decode_attention_flash_amd import synth
from gpu_common import DEV, counters_ready, note

pytestmark = pytest.mark.gpu

REPLAYS = 1000


def stress(B, Hq, Hkv, D, cap, lo, hi, num_splits, seed, n_q=1):
    k, v = synth.kv_cache(B, cap, Hkv, D, [cap] * B, seed, device=DEV, garbage=False)
    q = synth.queries(B, n_q, Hq, D, seed, device=DEV)
    shape = ck.shape_of(q, k)
    ws = ck.new_workspace(shape, num_splits=num_splits)
    lens_d = torch.full((B,), hi, dtype=torch.int32, device=DEV)
    out = torch.empty((B, n_q, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, n_q, Hq), dtype=torch.float32, device=DEV)
    eo = torch.empty_like(out)
    el = torch.empty_like(lse)

    def launch(o, l):
        ck.decode_attn(q, k, v, lens_d, causal=n_q > 1, out=o, lse=l, workspace=ws, num_splits=num_splits)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch(out, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    lens_all = torch.from_numpy(rng.integers(lo, hi + 1, size=(REPLAYS, B)).astype(np.int32)).to(DEV)
    note(f"stress B={B} n_q={n_q} D={D} cap={cap} splits={num_splits}: {REPLAYS} replays")
    for r in range(REPLAYS):
        lens_d.copy_(lens_all[r])
        graph.replay()
        launch(eo, el)
        if not (torch.equal(out, eo) and torch.equal(lse, el)):
            pytest.fail(f"replay {r} (lengths {lens_all[r].tolist()[:4]}...) differs from the eager launch")
    torch.cuda.synchronize()
    if ws is not None:
        assert ck.workspace_status(ws) == 0
        assert counters_ready(ws, ck.plan(shape, num_splits=num_splits)["units"])
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("num_splits", [0, 2, 7, 64])
def test_stress_d256_layer(num_splits):
    """The head_dim-256 layer (Hq=16, Hkv=4), lengths uniform in [1, 8192]."""
    stress(1, 16, 4, 256, 8192, 1, 8192, num_splits, 5100 + num_splits)


@pytest.mark.parametrize("num_splits", [0, 2, 7])
def test_stress_ragged_batch(num_splits):
    """The ragged batch shape (B=32, Hq=32, Hkv=8, D=128, capacity 32768),
    lengths uniform in [512, 32768]."""
    stress(32, 32, 8, 128, 32768, 512, 32768, num_splits, 5200 + num_splits)


@pytest.mark.parametrize("num_splits", [0, 3])
def test_stress_short_spans(num_splits):
    """Short sequences (B=2, Hq=8, Hkv=2, D=128, capacity 1024), lengths
    uniform in [1, 1024]: with automatic splits the lengths cross the
    single-split bound (256 positions) and the one-slice merge bound."""
    stress(2, 8, 2, 128, 1024, 1, 1024, num_splits, 5300 + num_splits)


@pytest.mark.parametrize("n_q", [3, 4, 6])
def test_stress_windows(n_q):
    """Causal windows over the head_dim-256 layer, lengths uniform in [1,
    8192]: n_q 3-4 cross the 6144-position bound of their split cap, n_q 6
    runs as two 16-row groups sharing tiles."""
    stress(1, 16, 4, 256, 8192, 1, 8192, 0, 5400 + n_q, n_q=n_q)
