"""Helpers shared by the GPU tests: run the HIP library and the oracle on the
same seeded inputs and compare them to the stated tolerances."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import decode_attention_flash_amd as ck
import oracle
from decode_attention_flash_amd import synth

# Tolerances for N(0, 1) inputs: max |delta| against the fp64 oracle.
TOL_F32 = 4e-3     # fp32 output
TOL_BF16 = 1.6e-2  # bf16 output (one bf16 rounding of values of magnitude < 4)
# lse: the row sum adds bf16-rounded weights (relative error <= 2^-8 each), so
# ln of it can move by at most ln(1 + 2^-8) < 4e-3.
TOL_LSE = 4e-3

DEV = torch.device("cuda", 0)


def note(msg: str) -> None:
    """Name the case before the GPU runs it (flushes through pytest capture)."""
    sys.__stdout__.write(f"[case] {msg}\n")
    sys.__stdout__.flush()


def dense_gpu(q, k, v, lens, *, causal=False, keep_mask=None, out_dtype=torch.float32,
              num_splits=0, scale=None, device_inputs=None):
    D = q.shape[-1]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    if device_inputs is None:
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    else:
        qd, kd, vd = device_inputs
    lens_d = torch.as_tensor(np.asarray(lens), dtype=torch.int32).to(DEV)
    mask_d = None if keep_mask is None else torch.as_tensor(np.asarray(keep_mask)).to(DEV)
    out, lse = ck.decode_attn(qd, kd, vd, lens_d, scale=scale, causal=causal, keep_mask=mask_d,
                              out_dtype=out_dtype, return_lse=True, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def gather_gpu(q, k, v, lens, idx, *, causal=False, out_dtype=torch.float32, num_splits=0,
               scale=None):
    D = q.shape[-1]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    lens_d = torch.as_tensor(np.asarray(lens), dtype=torch.int32).to(DEV)
    idx_d = torch.as_tensor(np.asarray(idx), dtype=torch.int32).to(DEV)
    out, lse = ck.decode_attn_gather(q.to(DEV), k.to(DEV), v.to(DEV), lens_d, idx_d, scale=scale,
                                     causal=causal, out_dtype=out_dtype, return_lse=True,
                                     num_splits=num_splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def oracle_ref(q, k, v, lens, *, causal=False, keep_mask=None, idx=None, scale=None):
    D = q.shape[-1]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    return oracle.attn(q, k, v, np.asarray(lens, dtype=np.int32), scale, causal,
                       keep_mask=keep_mask, idx=idx)


def steps_gpu(q, k, v, lens, ks, vs, *, out_dtype=torch.float32, num_splits=0, scale=None,
              device_inputs=None):
    D = q.shape[-1]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    if device_inputs is None:
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    else:
        qd, kd, vd = device_inputs
    lens_d = torch.as_tensor(np.asarray(lens), dtype=torch.int32).to(DEV)
    out, lse = ck.decode_attn_steps(qd, kd, vd, lens_d, ks.to(DEV), vs.to(DEV), scale=scale,
                                    out_dtype=out_dtype, return_lse=True, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def steps_ref(q, k, v, lens, ks, vs, *, scale=None):
    D = q.shape[-1]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    return oracle.attn_steps(q, k, v, np.asarray(lens, dtype=np.int32), ks, vs, scale)


def assert_close(gpu, ref, out_dtype=torch.float32, what=""):
    go, gl = gpu
    ro, rl = ref
    tol = TOL_BF16 if out_dtype == torch.bfloat16 else TOL_F32
    assert np.all(np.isfinite(go)), f"{what}: non-finite output"
    d = float(np.max(np.abs(go - ro))) if go.size else 0.0
    assert d <= tol, f"{what}: max|delta| {d:.3e} > {tol}"
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty), f"{what}: empty-row lse mismatch"
    if np.any(~empty):
        dl = float(np.max(np.abs(gl[~empty] - rl[~empty])))
        assert dl <= TOL_LSE, f"{what}: lse max|delta| {dl:.3e}"
    return d


def counting_case(n_q, Hq, Hkv, D, cap, lens, seed, nbits=17):
    B = len(lens)
    k, _ = synth.kv_cache(B, cap, Hkv, D, lens, seed)
    v1 = synth.counting_values(cap, Hkv, D, nbits)
    v = v1.expand(B, cap, Hkv, D).contiguous()
    for b, L in enumerate(lens):
        k[b, :L] = 0
        v[b, L:] = float("nan")
        k[b, L:] = float("nan")
    q = synth.queries(B, n_q, Hq, D, seed)
    return q, k, v


def check_counts(out, visible_sets, G, nbits=17):
    """out [B, n_q, Hq, D] fp32; visible_sets[b][i][g] = array of cells."""
    B, n_q, Hq, _ = out.shape
    for b in range(B):
        for i in range(n_q):
            for h in range(Hq):
                cells = np.asarray(visible_sets[b][i][h // G], dtype=np.int64)
                n = len(cells)
                if n == 0:
                    assert np.all(out[b, i, h] == 0.0)
                    continue
                o = out[b, i, h].astype(np.float64)
                assert abs(o[nbits] - 1.0) < 1e-6
                counts = np.array([np.sum((cells >> d) & 1) for d in range(nbits)])
                got = n * o[:nbits]
                assert np.max(np.abs(got - counts)) < 0.01, (b, i, h)
                assert np.array_equal(np.rint(got).astype(np.int64), counts), (b, i, h)


def counters_ready(ws: torch.Tensor, units: int) -> bool:
    """The workspace is ready for another launch of its plan: the status word
    (the first int32 of a 256-byte header) is 0, and for each unit (2 KiB of
    counters after the header: a parity word, then two sets of 128 ints) the
    set the parity names is all zero."""
    w = ws.view(torch.int32).cpu().numpy()
    if w[0] != 0:
        return False
    blk = w[64:64 + units * 512].reshape(units, 512)
    for u in range(units):
        par = int(blk[u, 0]) & 1
        if np.any(blk[u, 128 + 128 * par:256 + 128 * par] != 0):
            return False
    return True
