#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Headline workload: a full-attention layer of the Hq=16 / Hkv=4 / head_dim 256
shape at batch 1, one query, cache capacity 24007, kv_len 8000 (the shortest
length at which the dense path is held to 70 % of HBM peak).  A timed step
is one decode step through a stack of `layers` such layers, each with its own
KV cache, replayed from one HIP graph; `layers` is chosen so that a step reads
at least 1 GiB, which keeps the caches out of the 256 MB Infinity Cache.
value = microseconds per layer-step.  The kv_len sweep, the capacity sweep,
the causal window, the ragged batch and the gathered/masked sparse decode are
reported in the same JSON line under "sweep".

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "decode-attn µs/layer-step and achieved HBM GB/s (KV bytes read) vs kv_len"


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def layers_for(bytes_per_launch: int) -> int:
    return int(min(256, max(4, math.ceil((1 << 30) / max(1, bytes_per_launch)))))


class Stack:
    """`n` layers of K/V caches [B, cap, Hkv, D] bf16 ~ N(0, 1), on the device."""

    def __init__(self, n, B, cap, Hkv, D, seed):
        import torch
        self.k, self.v = [], []
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        for _ in range(n):
            self.k.append(torch.randn((B, cap, Hkv, D), generator=g, device="cuda",
                                      dtype=torch.bfloat16))
            self.v.append(torch.randn((B, cap, Hkv, D), generator=g, device="cuda",
                                      dtype=torch.bfloat16))


# per-replay times (ms) of the last time_graph call
LAST_REPLAYS_MS = []


def time_graph(launch_layer, n_layers, steps, warmup):
    """Capture n_layers launches in one graph; time `steps` replays.
    Returns (ms per replay, us per layer); the per-replay times are left in
    LAST_REPLAYS_MS."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for l in range(n_layers):
            launch_layer(l)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for l in range(n_layers):
            launch_layer(l)
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        graph.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[steps]) / steps
    LAST_REPLAYS_MS[:] = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    del graph
    return ms, ms * 1000.0 / n_layers


def replay_spread(n_layers):
    """p10 / median / p90 of the last time_graph call, in us per layer."""
    import numpy as np
    us = np.array(LAST_REPLAYS_MS) * 1000.0 / n_layers
    return {"us_p10": round(float(np.percentile(us, 10)), 3), "us_median": round(float(np.median(us)), 3),
            "us_p90": round(float(np.percentile(us, 90)), 3)}


def dense_case(stack, B, n_q, Hq, Hkv, D, lens, steps, warmup, causal=False, n_layers=None,
               masks=None, stamps=None):
    import torch
    import decode_attention_flash_amd as ck
    from decode_attention_flash_amd import synth
    cap = stack.k[0].shape[1]
    kv_bytes = int(sum(4 * Hkv * D * min(int(L), cap) for L in lens))
    window_bytes = kv_bytes
    if masks is not None:
        kv_bytes_mask = int(sum(n_q * Hkv * min(int(L), cap) for L in lens))
    else:
        kv_bytes_mask = 0
    n = n_layers or layers_for(kv_bytes)
    n = min(n, len(stack.k))
    qs = [synth.queries(B, n_q, Hq, D, 7 + l, device="cuda") for l in range(n)]
    outs = [torch.empty((B, n_q, Hq, D), dtype=torch.float32, device="cuda") for _ in range(n)]
    lens_d = torch.as_tensor(lens, dtype=torch.int32, device="cuda")
    shape = ck.shape_of(qs[0], stack.k[0])
    ws = ck.new_workspace(shape)
    if masks is not None and cap % 16 == 0 and all(m.data_ptr() % 16 == 0 for m in masks[:n]):
        # The scan reads only the tiles that hold a kept cell of the unit's
        # query rows (rows below the length), so count those, per layer.
        kv_bytes = int(sum(masked_read_tokens(masks[l], lens, ck.plan(shape)["tile"]) for l in range(n)) * 4 * D / n)

    grid = 0
    if stamps is not None:  # phase timestamps: one block of workgroups per layer
        pl = ck.plan(shape)
        grid = pl["units"] * pl["splits"]
        assert pl["row_groups"] == 1 and stamps.shape[0] >= n * grid

    def launch(l):
        if stamps is not None:
            ck.set_phase_stamps(stamps[l * grid:(l + 1) * grid])
        ck.decode_attn(qs[l], stack.k[l], stack.v[l], lens_d, causal=causal, out=outs[l],
                       workspace=ws, keep_mask=None if masks is None else masks[l])

    try:
        ms, us = time_graph(launch, n, steps, warmup)
    finally:
        if stamps is not None:
            ck.set_phase_stamps(None)
    algo = kv_bytes + kv_bytes_mask + 2 * B * n_q * Hq * D + 4 * B * n_q * Hq * D + 4 * B
    res = dict(us=us, ms_per_replay=ms, layers=n, kv_bytes=kv_bytes, algo_bytes=algo,
               kv_gbs=kv_bytes / us / 1e3, algo_gbs=algo / us / 1e3,
               frac_kv=kv_bytes / us / 1e3 / PEAK_HBM_GBS, **replay_spread(n))
    if masks is not None:
        res["window_bytes"] = window_bytes
    if stamps is not None:
        res["grid"] = grid
    return res


PHASES = ["length known", "first tile loaded", "tile loop done", "all waves done", "partial stored",
          "arrived"]


def phase_breakdown(stamps, n, grid):
    """Per launch, times (us) from the first workgroup's start to each phase:
    median and last over the active splits, then the median of those over
    the launches.  The counter runs at 100 MHz."""
    import numpy as np
    a = stamps[:n * grid].cpu().numpy().reshape(n, grid, 16)
    per = []
    for l in range(n):
        t = a[l]
        meta = t[:, 15]
        s = meta & 0xFFFF
        n_active = (meta >> 32) & 0xFFFF
        role = (meta >> 48) & 0xFF
        rel = (t - t[:, 0].min()).astype(np.float64) / 100.0
        act = s < n_active
        row = {"last start": rel[:, 0].max()}
        for k, name in enumerate(PHASES, start=1):
            if k >= 5 and not np.any(n_active[act] > 1):
                continue
            row[name + " (median)"] = float(np.median(rel[act, k]))
            row[name + " (last)"] = float(rel[act, k].max())
        merging = act & ((role == 1) | (role == 2))
        if np.any(merging):
            row["merge begins (median)"] = float(np.median(rel[merging, 7]))
            row["merge ends (last)"] = float(rel[merging, 8].max())
            row["merging workgroups"] = int(np.sum(merging))
            row["slices per last arrival"] = float(np.mean(t[act & (role == 1), 13]))
            last, helper = act & (role == 1), act & (role == 2)
            row["last arrival's merge and claims"] = float(np.mean(rel[last, 8] - rel[last, 7]))
            if np.any(helper):
                row["helper start after last arrival"] = float(np.mean(rel[helper, 7]) - rel[last, 6].max())
                row["helper merge"] = float(np.mean(rel[helper, 8] - rel[helper, 7]))
                row["helpers end (last)"] = float(rel[helper, 8].max())
            row["last arrivals end (last)"] = float(rel[last, 8].max())
        else:
            row["output stored (last)"] = float(rel[act, 5].max())
        row["active workgroups"] = int(np.sum(act))
        per.append(row)
    keys = per[0].keys()
    return {k: float(np.median([r[k] for r in per if k in r])) for k in keys}


def masked_read_tokens(mask, lens, tile):
    """Cache positions a tile-skipping scan reads, summed over (sequence, KV
    head): those below the length in tiles where some query row keeps a
    cell.  mask [B, n_q, Hkv, cap] on the device."""
    import torch
    total = 0
    for b, L in enumerate(lens):
        L = min(int(L), mask.shape[-1])
        if L == 0:
            continue
        keep = (mask[b, :, :, :L] != 0).any(dim=0)  # [Hkv, L]
        nt = -(-L // tile)
        keep = torch.nn.functional.pad(keep, (0, nt * tile - L)).view(keep.shape[0], nt, tile).any(-1)
        last = L - (nt - 1) * tile  # positions of the last tile below the length
        total += int(keep[:, :-1].sum().item()) * tile + int(keep[:, -1].sum().item()) * last
    return total


def steps_case(stack, n_q, Hq, Hkv, D, L, steps, warmup, n_layers=None):
    """Verification window with the drafts beside the cache (decode_attn_steps)."""
    import torch
    import decode_attention_flash_amd as ck
    from decode_attention_flash_amd import synth
    kv_bytes = 4 * Hkv * D * (L + n_q)
    n = min(n_layers or layers_for(kv_bytes), len(stack.k))
    qs = [synth.queries(1, n_q, Hq, D, 9 + l, device="cuda") for l in range(n)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    kss = [torch.randn((1, n_q, Hkv, D), generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(n)]
    vss = [torch.randn((1, n_q, Hkv, D), generator=gen, device="cuda", dtype=torch.bfloat16) for _ in range(n)]
    outs = [torch.empty((1, n_q, Hq, D), dtype=torch.float32, device="cuda") for _ in range(n)]
    lens_d = torch.tensor([L], dtype=torch.int32, device="cuda")
    ws = ck.new_workspace(ck.shape_of(qs[0], stack.k[0]))

    def launch(l):
        ck.decode_attn_steps(qs[l], stack.k[l], stack.v[l], lens_d, kss[l], vss[l], out=outs[l], workspace=ws)

    ms, us = time_graph(launch, n, steps, warmup)
    return dict(us=us, ms_per_replay=ms, layers=n, kv_bytes=kv_bytes, kv_gbs=kv_bytes / us / 1e3,
                frac_kv=kv_bytes / us / 1e3 / PEAK_HBM_GBS)


class Q8Stack:
    """`n` layers of paged INT8 caches (random codes and scales, the block
    tables a random permutation of each layer's pool), on the device."""

    def __init__(self, n, B, cap, Hkv, D, page, seed):
        import torch
        import decode_attention_flash_amd as ck
        self.caches = []
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        max_pages = (cap + page - 1) // page
        for _ in range(n):
            perm = torch.randperm(B * max_pages, generator=g, device="cuda").to(torch.int32)
            c = ck.PagedQ8Cache(B * max_pages, page, Hkv, D, perm.view(B, max_pages))
            c.k_codes.copy_(torch.randint(-127, 128, c.k_codes.shape, generator=g, device="cuda",
                                          dtype=torch.int8))
            c.v_codes.copy_(torch.randint(-127, 128, c.v_codes.shape, generator=g, device="cuda",
                                          dtype=torch.int8))
            c.k_scales.uniform_(0.005, 0.03, generator=g)
            c.v_scales.uniform_(0.005, 0.03, generator=g)
            self.caches.append(c)


def q8_case(stack, B, n_q, Hq, Hkv, D, lens, steps, warmup, causal=False, n_layers=None):
    """Decode over the paged INT8 cache (decode_attn_q8); bytes read are the
    int8 codes plus one fp32 scale per token row, for K and V."""
    import torch
    import decode_attention_flash_amd as ck
    from decode_attention_flash_amd import synth
    kv_bytes = int(sum(2 * Hkv * (D + 4) * int(L) for L in lens))
    n = min(n_layers or layers_for(kv_bytes), len(stack.caches))
    qs = [synth.queries(B, n_q, Hq, D, 13 + l, device="cuda") for l in range(n)]
    outs = [torch.empty((B, n_q, Hq, D), dtype=torch.float32, device="cuda") for _ in range(n)]
    lens_d = torch.as_tensor(lens, dtype=torch.int32, device="cuda")
    c0 = stack.caches[0]
    ws = ck.new_workspace(ck.Shape(B, n_q, Hq, Hkv, D, c0.capacity))

    def launch(l):
        ck.decode_attn_q8(qs[l], stack.caches[l], lens_d, causal=causal, out=outs[l], workspace=ws)

    ms, us = time_graph(launch, n, steps, warmup)
    return dict(us=us, ms_per_replay=ms, layers=n, kv_bytes=kv_bytes, kv_gbs=kv_bytes / us / 1e3,
                frac_kv=kv_bytes / us / 1e3 / PEAK_HBM_GBS)


def gather_case(stack, n_kv, W_sel, tail, steps, warmup, n_layers=None, block=0):
    """Gather over per-layer top-k lists of W_sel cells plus the tail: cells
    drawn one by one, or (block > 0) as W_sel / block aligned runs."""
    import numpy as np
    import torch
    import decode_attention_flash_amd as ck
    from decode_attention_flash_amd import synth
    B, n_q, Hq, Hkv, D = 1, 1, 16, 2, 128
    W = W_sel + tail
    kv_bytes = B * n_q * Hkv * W * 4 * D
    n = min(n_layers or layers_for(kv_bytes), len(stack.k))
    qs = [synth.queries(B, n_q, Hq, D, 11 + l, device="cuda") for l in range(n)]
    outs = [torch.empty((B, n_q, Hq, D), dtype=torch.float32, device="cuda") for _ in range(n)]
    def lists(l):
        if block:
            return synth.block_lists(B, n_q, Hkv, n_kv, W_sel // block, block, tail, seed=5100 + n_kv + l)
        return synth.topk_lists(B, n_q, Hkv, n_kv, W_sel, tail, seed=5000 + n_kv + l)

    idxs = [torch.from_numpy(lists(l)).to("cuda") for l in range(n)]
    lens_d = torch.full((B,), n_kv, dtype=torch.int32, device="cuda")
    shape = ck.shape_of(qs[0], stack.k[0])
    ws = ck.new_workspace(shape, W=W)

    def launch(l):
        ck.decode_attn_gather(qs[l], stack.k[l], stack.v[l], lens_d, idxs[l], out=outs[l],
                              workspace=ws)

    ms, us = time_graph(launch, n, steps, warmup)
    algo = kv_bytes + 4 * W * Hkv + 6 * B * n_q * Hq * D + 4
    return dict(us=us, ms_per_replay=ms, layers=n, kv_bytes=kv_bytes, algo_bytes=algo,
                kv_gbs=kv_bytes / us / 1e3, frac_kv=kv_bytes / us / 1e3 / PEAK_HBM_GBS), idxs


def topk_case(B, n_q, Hs, cap, lens, k, tail, steps, warmup, with_gather=None):
    """Top-k index lists over per-layer score buffers (decode_topk); with
    with_gather = (stack, Hq, D), each layer's lists also feed the gathered
    attention in the same graph (the whole sparse step of a layer)."""
    import torch
    import decode_attention_flash_amd as ck
    from decode_attention_flash_amd import synth
    score_bytes = B * n_q * Hs * cap * 4
    n = layers_for(score_bytes)
    if with_gather is not None:
        n = min(n, len(with_gather[0].k))
    scs = [synth.index_scores(B, n_q, Hs, cap, 90 + l, device="cuda") for l in range(n)]
    lens_d = torch.as_tensor(lens, dtype=torch.int32, device="cuda")
    idxs = [torch.empty((B, n_q, Hs, k + tail), dtype=torch.int32, device="cuda") for _ in range(n)]
    if with_gather is None:
        def launch(l):
            ck.decode_topk(scs[l], lens_d, k, tail=tail, out=idxs[l])
    else:
        st, Hq, D = with_gather
        qs = [synth.queries(B, n_q, Hq, D, 13 + l, device="cuda") for l in range(n)]
        outs = [torch.empty((B, n_q, Hq, D), dtype=torch.float32, device="cuda") for _ in range(n)]
        ws = ck.new_workspace(ck.shape_of(qs[0], st.k[0]), W=k + tail)

        def launch(l):
            ck.decode_topk(scs[l], lens_d, k, tail=tail, out=idxs[l])
            ck.decode_attn_gather(qs[l], st.k[l], st.v[l], lens_d, idxs[l], out=outs[l], workspace=ws)
    ms, us = time_graph(launch, n, steps, warmup)
    _, us_torch = time_graph(lambda l: torch.topk(scs[l][..., :int(max(lens)) - tail], k, dim=-1, sorted=False),
                             n, steps, warmup)
    P = ck.topk_plan((B, n_q, Hs, cap), k, tail)["wgs_per_row"]
    return dict(us=us, ms_per_replay=ms, layers=n, score_bytes=score_bytes, wgs_per_row=P,
                torch_topk_us=us_torch)


def calibrate_copy(nbytes: int = 1 << 28, reps: int = 3) -> None:
    """A plain device copy of known size, so that a counter profile of this
    run can scale its byte counters (FETCH_SIZE / WRITE_SIZE) against it."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def kernel_source_digest() -> str:
    import hashlib
    path = os.path.join(ROOT, "decode_attention_flash_amd", "csrc", "ck_decode_attn.hip")
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source for this workload; else None."""
    path = os.path.join(ROOT, "profiles", "decode_kernel_d256_traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != kernel_source_digest() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def host_info() -> dict:
    """Host CPU facts for the CPU-baseline record."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count()
    return {"host_nproc": os.cpu_count(), "host_cpus_allowed": allowed, "cpu_model": model}


def _time_calls(fn, seconds: float) -> tuple[float, int]:
    """Mean seconds per call of fn over at least `seconds` (one call at least)."""
    fn()  # warm
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return el / reps, reps


def cpu_baseline(seconds: float):
    """The oracle on the host cores, beside each workload: a full layer-step
    where it finishes in time, else a stated sample scaled to one layer-step;
    timed with every allowed host core (capped by OMP_NUM_THREADS) and with
    one thread.  `seconds` is the time per (workload, thread count)."""
    import numpy as np
    import oracle
    from decode_attention_flash_amd import synth
    threads = oracle.default_threads()
    cases = []
    # tiny decode: B=1, Hq=8, Hkv=2, D=128, cap 1024, kv_len 300
    k, v = synth.kv_cache(1, 1024, 2, 128, [300], 1001)
    q = synth.queries(1, 1, 8, 128, 1001)
    cases.append(("tiny decode B=1 Hq=8 Hkv=2 D=128 kv_len=300", 1.0, "full layer-step",
                  lambda nt: oracle.attn(q, k, v, np.array([300], np.int32), 1 / math.sqrt(128), nthreads=nt)))
    # the headline layer: B=1, Hq=16, Hkv=4, D=256, cap 24007, kv_len 8000
    k2, v2 = synth.kv_cache(1, 24007, 4, 256, [8000], 1002)
    q2 = synth.queries(1, 1, 16, 256, 1002)
    cases.append(("D=256 layer B=1 Hq=16 Hkv=4 kv_len=8000 cap=24007", 1.0, "full layer-step",
                  lambda nt: oracle.attn(q2, k2, v2, np.array([8000], np.int32), 1 / math.sqrt(256), nthreads=nt)))
    # ragged batch: 4 of the 32 sequences, scaled by the batch's total length
    lens = synth.ragged_lens(32, 512, 32768, 4000)
    pick = [0, 8, 16, 24]
    ls = lens[pick].astype(np.int32)
    k4, v4 = synth.kv_cache(len(pick), int(ls.max()), 8, 128, ls, 1004, garbage=False)
    q4 = synth.queries(len(pick), 1, 32, 128, 1004)
    cases.append(("ragged batch B=32 Hq=32 Hkv=8 D=128 cap=32768", float(lens.sum()) / float(ls.sum()),
                  f"sequences {pick} (kv_len {ls.tolist()}), scaled by total kv_len {int(lens.sum())}",
                  lambda nt: oracle.attn(q4, k4, v4, ls, 1 / math.sqrt(128), nthreads=nt)))
    # sparse decode: 2048 + 64 gathered cells per KV head out of 131072
    k5, v5 = synth.kv_cache(1, 131072, 2, 128, [131072], 1005)
    q5 = synth.queries(1, 1, 16, 128, 1005)
    idx5 = synth.topk_lists(1, 1, 2, 131072, 2048, 64, seed=5000 + 131072)
    cases.append(("gathered sparse decode B=1 Hq=16 Hkv=2 D=128 n_kv=131072 W=2112", 1.0, "full layer-step",
                  lambda nt: oracle.attn(q5, k5, v5, np.array([131072], np.int32), 1 / math.sqrt(128),
                                         idx=idx5, nthreads=nt)))
    per = max(0.5, seconds / (2 * len(cases)))
    rows = []
    for name, scale_to_step, sample, fn in cases:
        t_multi, r_multi = _time_calls(lambda: fn(threads), per)
        t_single, r_single = _time_calls(lambda: fn(1), per)
        rows.append({"workload": name, "sample": sample, "threads": threads,
                     "us_per_layer_step": round(t_multi * scale_to_step * 1e6, 1),
                     "us_per_layer_step_1_thread": round(t_single * scale_to_step * 1e6, 1),
                     "calls": [r_multi, r_single]})
    head = rows[1]
    return {"value": head["us_per_layer_step"], "unit": "us/layer-step", "cores": threads, "kind": "oracle",
            "sample": f"full layer-steps of the headline workload ({head['workload']}), fp64, {threads} threads; "
                      "the other workloads in 'configs'",
            "threads": threads, "single_thread_value": head["us_per_layer_step_1_thread"],
            **host_info(), "configs": rows}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kv-len", type=int, default=8000)
    ap.add_argument("--headline-only", action="store_true", help="skip the sweeps and the CPU leg")
    ap.add_argument("--only", default="",
                    help="comma-separated sweep groups to run (dense, sparse, topk, q8, contraction; "
                         "window: only the n_q=6 causal window at kv_len 4000, for counter profiles); "
                         "skips the CPU leg")
    ap.add_argument("--cases", default="",
                    help="with the contraction group: comma-separated cases to run (tiny, 1000, 8000, 24000, "
                         "ragged, gather32768, gather131072; default all)")
    ap.add_argument("--phases", action="store_true",
                    help="also record phase timestamps of the head_dim-256 layer at kv_len 1000, 8000, 24000")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="oracle timing budget (split over four workloads, multi- and single-threaded)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device copy (reference for counter profiles)")
    args = ap.parse_args()
    groups = {"dense", "sparse", "topk", "q8"}
    if args.headline_only:
        groups = set()
    elif args.only:
        groups = {g.strip() for g in args.only.split(",") if g.strip()}
        unknown = groups - {"dense", "sparse", "topk", "q8", "window", "contraction"}
        if unknown:
            ap.error(f"unknown sweep groups: {sorted(unknown)}")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library's kernels run on a single device "
              "and there is no multi-GPU path to time (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_flash_amd as ck
    ck.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    Hq, Hkv, D, cap = 16, 4, 256, 24007
    L0 = args.kv_len
    lens_sweep = [1000, 3000, 8000, 24000]
    n_max = max(layers_for(4 * Hkv * D * L) for L in lens_sweep + [L0]) if "dense" in groups else 4
    n_max = max(n_max, layers_for(4 * Hkv * D * L0))
    if args.phases:
        n_max = max(n_max, layers_for(4 * Hkv * D * 1000))
    log(f"allocating {n_max} layer caches of capacity {cap}")
    stack = Stack(n_max, 1, cap, Hkv, D, 1002)

    log(f"headline: kv_len={L0}")
    head = dense_case(stack, 1, 1, Hq, Hkv, D, [L0], args.steps, args.warmup)
    log(f"headline: {head['us']:.2f} us/layer-step, {head['kv_gbs']:.0f} GB/s on KV bytes")

    if args.calibrate_copy:
        calibrate_copy()

    phases = None
    if args.phases:
        phases = []
        for L in (1000, 8000, 24000):
            n = min(layers_for(4 * Hkv * D * L), len(stack.k))
            pl = ck.plan(ck.Shape(1, 1, Hq, Hkv, D, cap))
            stamps = torch.zeros((n * pl["units"] * pl["splits"], 16), dtype=torch.int64, device="cuda")
            r = dense_case(stack, 1, 1, Hq, Hkv, D, [L], args.steps, args.warmup, n_layers=n, stamps=stamps)
            b = phase_breakdown(stamps, r["layers"], r["grid"])
            log(f"phases kv_len {L} ({r['us']:.2f} us/layer with stamps on): " +
                ", ".join(f"{k} {v:.0f}" if k.endswith("workgroups") else f"{k} {v:.2f}"
                          for k, v in b.items()))
            phases.append(dict(kv_len=L, us_stamped=r["us"], **b))
            del stamps

    sweep = {}
    if "window" in groups:
        # 24 packed rows on 4 KV heads: two 16-row groups per head sharing tiles
        r = dense_case(stack, 1, 6, Hq, Hkv, D, [4000], args.steps, args.warmup, causal=True)
        log(f"window n_q=6 L=4000: {r['us']:.2f} us")
        sweep["window_n6"] = dict(kv_len=4000, n_q=6, **r)
    if "dense" in groups:
        sweep["kv_len"] = []
        for L in lens_sweep:
            r = dense_case(stack, 1, 1, Hq, Hkv, D, [L], args.steps, args.warmup)
            log(f"kv_len {L}: {r['us']:.2f} us, {r['kv_gbs']:.0f} GB/s")
            sweep["kv_len"].append(dict(kv_len=L, cap=cap, **r))
        # cost against length: least-squares line us = intercept + bytes / rate
        import numpy as np
        xb = np.array([e["kv_bytes"] for e in sweep["kv_len"]], dtype=np.float64)
        yu = np.array([e["us"] for e in sweep["kv_len"]], dtype=np.float64)
        slope, icpt = np.polyfit(xb, yu, 1)
        sweep["kv_len_fit"] = {"intercept_us": round(float(icpt), 2),
                               "marginal_gbs": round(float(1e-3 / slope), 1)}
        log(f"kv_len fit: intercept {icpt:.2f} us, marginal {1e-3 / slope:.0f} GB/s")
        # warm: the kv_len-8000 layer with every launch on one cache (it
        # stays in the 256 MB Infinity Cache); labelled, never the headline
        warm = Stack.__new__(Stack)
        warm.k, warm.v = [stack.k[0]] * 33, [stack.v[0]] * 33
        r = dense_case(warm, 1, 1, Hq, Hkv, D, [8000], args.steps, args.warmup, n_layers=33)
        log(f"warm (one cache) kv_len 8000: {r['us']:.2f} us")
        sweep["warm_kv_len_8000"] = dict(kv_len=8000, cap=cap, note="one cache replayed (warm)", **r)
        sweep["causal_window"] = []
        for L in (2000, 4000):
            # the same bytes as one query: the window's cost against it
            r1 = dense_case(stack, 1, 1, Hq, Hkv, D, [L], args.steps, args.warmup)
            log(f"window n_q=1 L={L}: {r1['us']:.2f} us")
            sweep["causal_window"].append(dict(kv_len=L, n_q=1, ratio_vs_nq1=1.0, **r1))
            for n_q in (3, 4, 5, 6):
                r = dense_case(stack, 1, n_q, Hq, Hkv, D, [L], args.steps, args.warmup, causal=True)
                ratio = r["us"] / r1["us"]
                log(f"window n_q={n_q} L={L}: {r['us']:.2f} us ({ratio:.2f}x n_q=1)")
                sweep["causal_window"].append(dict(kv_len=L, n_q=n_q, ratio_vs_nq1=round(ratio, 3), **r))
        sweep["step_rows"] = []
        for L in (2000, 4000):
            for n_q in (3, 4, 5, 6):
                r = steps_case(stack, n_q, Hq, Hkv, D, L - n_q, args.steps, args.warmup)
                log(f"step rows n_q={n_q} prefix={L - n_q}: {r['us']:.2f} us")
                sweep["step_rows"].append(dict(prefix=L - n_q, n_q=n_q, **r))
        del stack
        torch.cuda.empty_cache()
        # short sequences: the tiny decode layer (Hq=8, Hkv=2, D=128, capacity
        # 1024) and the head_dim-256 layer at 100 tokens
        sweep["short"] = []
        st = Stack(256, 1, 1024, 2, 128, 1001)
        for L in (100, 300, 1000):
            r = dense_case(st, 1, 1, 8, 2, 128, [L], args.steps, args.warmup)
            log(f"short D=128 kv_len {L}: {r['us']:.2f} us")
            sweep["short"].append(dict(D=128, Hq=8, Hkv=2, cap=1024, kv_len=L, **r))
        del st
        st = Stack(256, 1, 1024, Hkv, D, 1002)
        r = dense_case(st, 1, 1, Hq, Hkv, D, [100], args.steps, args.warmup)
        log(f"short D=256 kv_len 100: {r['us']:.2f} us")
        sweep["short"].append(dict(D=D, Hq=Hq, Hkv=Hkv, cap=1024, kv_len=100, **r))
        del st
        torch.cuda.empty_cache()
        sweep["capacity"] = []
        for c in (8199, 16263, 24007):
            n = layers_for(4 * Hkv * D * 3000)
            st = Stack(n, 1, c, Hkv, D, 2000 + c)
            r = dense_case(st, 1, 1, Hq, Hkv, D, [3000], args.steps, args.warmup)
            log(f"cap {c} L=3000: {r['us']:.2f} us")
            sweep["capacity"].append(dict(kv_len=3000, cap=c, **r))
            del st
            torch.cuda.empty_cache()
        # ragged batch: B=32, Hq=32, Hkv=8, D=128, capacity 32768
        from decode_attention_flash_amd import synth
        lens = synth.ragged_lens(32, 512, 32768, 4000)
        st = Stack(4, 32, 32768, 8, 128, 1004)
        r = dense_case(st, 32, 1, 32, 8, 128, lens.tolist(), max(3, args.steps // 4), 2, n_layers=4)
        log(f"ragged B=32: {r['us']:.1f} us, {r['kv_gbs']:.0f} GB/s")
        sweep["ragged_batch"] = dict(B=32, sum_kv_len=int(lens.sum()), **r)
        del st
        torch.cuda.empty_cache()
    if "sparse" in groups:
        from decode_attention_flash_amd import synth
        # sparse: gathered top-k lists vs the masked full-window scan, with the
        # 2048 cells drawn one by one or as 32 aligned runs of 64 (tiles skip)
        sweep["sparse"] = []
        for n_kv in (32768, 65536, 131072):
            W_sel, tail = 2048, 64
            n_g = layers_for(2 * (W_sel + tail) * 4 * 128)
            n_m = layers_for(4 * 2 * 128 * n_kv)
            st = Stack(max(n_g, n_m), 1, n_kv, 2, 128, 1005)
            path = ck.sparse_path(ck.Shape(1, 1, 16, 2, 128, n_kv), W_sel + tail, n_kv)
            for block in (0, 64):
                sel = "blocks" if block else "scattered"
                rg, idxs = gather_case(st, n_kv, W_sel, tail, args.steps, args.warmup, block=block)
                masks = [torch.from_numpy(synth.mask_from_lists(idxs[l].cpu().numpy(), n_kv)).to("cuda")
                         for l in range(n_m)]
                rm = dense_case(st, 1, 1, 16, 2, 128, [n_kv], args.steps, args.warmup, n_layers=n_m,
                                masks=masks)
                log(f"sparse n_kv={n_kv} {sel}: gather {rg['us']:.2f} us, masked {rm['us']:.2f} us "
                    f"(chosen: {path})")
                sweep["sparse"].append(dict(n_kv=n_kv, selection=sel, chosen=path, gather=rg, masked=rm))
                del masks
            # the whole sparse step of a layer: top-k lists from scores, then the gather
            rs = topk_case(1, 1, 2, n_kv, [n_kv], W_sel, tail, args.steps, args.warmup,
                           with_gather=(st, 16, 128))
            log(f"sparse n_kv={n_kv}: top-k + gather {rs['us']:.2f} us")
            sweep["sparse"].append(dict(n_kv=n_kv, selection="top-k of scores", select_and_gather=rs))
            del st
            torch.cuda.empty_cache()

    if "topk" in groups:
        # top-k index lists from one score per cell: the sparse workload's two
        # rows (2048 + 64 cells), then selection and gathered attention as one
        # step, and a large batch (one workgroup per row)
        from decode_attention_flash_amd import synth
        sweep["topk"] = []
        for n_kv in (32768, 65536, 131072):
            r = topk_case(1, 1, 2, n_kv, [n_kv], 2048, 64, args.steps, args.warmup)
            log(f"top-k n_kv={n_kv}: {r['us']:.2f} us (torch.topk {r['torch_topk_us']:.2f})")
            sweep["topk"].append(dict(n_kv=n_kv, k=2048, tail=64, **r))
        lens = synth.ragged_lens(32, 512, 32768, 4000)
        r = topk_case(32, 1, 8, 32768, lens.tolist(), 2048, 64, args.steps, args.warmup)
        log(f"top-k B=32 x 8 heads: {r['us']:.2f} us (torch.topk {r['torch_topk_us']:.2f})")
        sweep["topk_batch"] = dict(B=32, Hs=8, cap=32768, k=2048, tail=64, **r)

    if "q8" in groups:
        # paged INT8 cache: the same head_dim-256 layer and the ragged batch
        sweep["q8_kv_len"] = []
        n_q8 = max(layers_for(2 * Hkv * (D + 4) * L) for L in lens_sweep)
        qst = Q8Stack(n_q8, 1, cap, Hkv, D, 128, 3001)
        for L in lens_sweep:
            r = q8_case(qst, 1, 1, Hq, Hkv, D, [L], args.steps, args.warmup)
            log(f"int8 pages kv_len {L}: {r['us']:.2f} us, {r['kv_gbs']:.0f} GB/s")
            sweep["q8_kv_len"].append(dict(kv_len=L, page=128, **r))
        sweep["q8_causal_window"] = []
        for L in (2000, 4000):
            for n_q in (3, 4, 5, 6):
                r = q8_case(qst, 1, n_q, Hq, Hkv, D, [L], args.steps, args.warmup, causal=True)
                log(f"int8 pages window n_q={n_q} L={L}: {r['us']:.2f} us")
                sweep["q8_causal_window"].append(dict(kv_len=L, n_q=n_q, page=128, **r))
        del qst
        torch.cuda.empty_cache()
        from decode_attention_flash_amd import synth
        lens = synth.ragged_lens(32, 512, 32768, 4000)
        qst = Q8Stack(4, 32, 32768, 8, 128, 128, 3004)
        r = q8_case(qst, 32, 1, 32, 8, 128, lens.tolist(), max(3, args.steps // 4), 2, n_layers=4)
        log(f"int8 pages ragged B=32: {r['us']:.1f} us, {r['kv_gbs']:.0f} GB/s")
        sweep["q8_ragged_batch"] = dict(B=32, sum_kv_len=int(lens.sum()), page=128, **r)
        del qst
        torch.cuda.empty_cache()

    if "contraction" in groups:
        # The workloads of at most 8 packed rows through the three
        # contractions, each case timed MFMA, VALU dot2, VALU fp32 on the
        # same caches.
        from decode_attention_flash_amd import synth
        sweep["contraction"] = []
        all_cases = ["tiny", "1000", "8000", "24000", "ragged", "gather32768", "gather131072"]
        cases = [c.strip() for c in args.cases.split(",") if c.strip()] or all_cases
        if set(cases) - set(all_cases):
            ap.error(f"unknown contraction cases: {sorted(set(cases) - set(all_cases))}")

        def both(name, run):
            res = {}
            for kind in ("mfma", "valu", "valu_f32"):
                ck.set_contraction(kind)
                try:
                    res[kind] = run()
                finally:
                    ck.set_contraction("mfma")
            log(f"contraction {name}: " + ", ".join(f"{k} {v['us']:.2f} us" for k, v in res.items()))
            sweep["contraction"].append(dict(case=name, **res))

        if "tiny" in cases:
            st = Stack(layers_for(4 * 2 * 128 * 300), 1, 1024, 2, 128, 1001)
            both("tiny B=1 Hq=8 Hkv=2 D=128 cap=1024 kv_len=300",
                 lambda: dense_case(st, 1, 1, 8, 2, 128, [300], args.steps, args.warmup))
            del st
        d256 = [L for L in (1000, 8000, 24000) if str(L) in cases]
        if d256:
            st = Stack(max(layers_for(4 * Hkv * D * L) for L in d256), 1, cap, Hkv, D, 1002)
            for L in d256:
                both(f"B=1 Hq={Hq} Hkv={Hkv} D={D} cap={cap} kv_len={L}",
                     lambda: dense_case(st, 1, 1, Hq, Hkv, D, [L], args.steps, args.warmup))
            del st
            torch.cuda.empty_cache()
        if "ragged" in cases:
            lens = synth.ragged_lens(32, 512, 32768, 4000)
            st = Stack(4, 32, 32768, 8, 128, 1004)
            both("ragged B=32 Hq=32 Hkv=8 D=128 cap=32768",
                 lambda: dense_case(st, 32, 1, 32, 8, 128, lens.tolist(), max(3, args.steps // 4), 2,
                                    n_layers=4))
            del st
            torch.cuda.empty_cache()
        for n_kv in (32768, 131072):
            if f"gather{n_kv}" not in cases:
                continue
            st = Stack(layers_for(2 * 2112 * 4 * 128), 1, n_kv, 2, 128, 1005)
            both(f"gather B=1 Hq=16 Hkv=2 D=128 n_kv={n_kv} W=2048+64",
                 lambda: gather_case(st, n_kv, 2048, 64, args.steps, args.warmup)[0])
            del st
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu and not args.headline_only and not args.only:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(args.cpu_seconds)

    workload = (f"decode layer B=1 n_q=1 Hq={Hq} Hkv={Hkv} D={D} cap={cap} kv_len={L0}, "
                f"{head['layers']} layer caches per step (cold)")
    traffic = measured_traffic(f"B=1 n_q=1 Hq={Hq} Hkv={Hkv} D={D} cap={cap} kv_len={L0}")
    line = {
        "metric": METRIC,
        "value": round(head["us"], 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_replay"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload,
                   "B": 1, "n_q": 1, "Hq": Hq, "Hkv": Hkv, "D": D, "cap": cap, "kv_len": L0,
                   "layers_per_step": head["layers"], "parallelism": "none"},
        "spread_us": {k: head[k] for k in ("us_p10", "us_median", "us_p90")},
        "hbm_gbs_kv": round(head["kv_gbs"], 1),
        "frac_of_peak_kv": round(head["frac_kv"], 4),
        "roofline": {"bound": "hbm", "achieved": round(head["algo_gbs"], 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(head["algo_gbs"] / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": "decode_kernel<256,1,0,false,0,false,false>",
                     "algo_bytes_per_launch": head["algo_bytes"]},
        "cpu_baseline": cpu,
        "sweep": sweep,
        "phases": phases,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
