"""Pins for the CPU fp64 oracle (CPU only).

The pages print no worked numeric example, so the oracle is pinned by a
library routine (torch SDPA in float64), closed forms and invariants; see
tests/oracle_pins.py.  The mutation test at the end plants plausible
mistakes in copies of the oracle source and checks that these pins catch
every one of them.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import oracle_pins as pins
from decode_attention_flash_amd import synth


@pytest.mark.parametrize("name", sorted(pins.ALL_CHECKS))
def test_pin(name):
    dev = pins.ALL_CHECKS[name](oracle.load())
    assert dev <= pins.TOL, f"{name}: deviation {dev}"


def test_garbage_and_capacity_do_not_change_result():
    """Output is bit-identical when the capacity grows or garbage is written
    past the filled length: the oracle never reads those cells."""
    B, n_q, Hq, Hkv, D = 2, 2, 4, 2, 32
    lens = np.array([50, 17], dtype=np.int32)
    q = synth.queries(B, n_q, Hq, D, 3)
    ref = None
    for cap, garbage in ((64, True), (64, False), (200, True)):
        k, v = synth.kv_cache(B, cap, Hkv, D, lens, 99, garbage=garbage)
        o, l = oracle.attn(q, k, v, lens, 0.2, True)
        if ref is None:
            ref = (o, l)
        else:
            assert np.array_equal(o, ref[0]) and np.array_equal(l, ref[1])
    # NaN garbage everywhere past L still leaves every output finite
    k, v = synth.kv_cache(B, 64, Hkv, D, lens, 99)
    k[:, 60:] = float("nan")
    v[:, 60:] = float("nan")
    o, _ = oracle.attn(q, k, v, lens, 0.2, True)
    assert np.all(np.isfinite(o))


def test_kv_lens_clamped_to_capacity():
    B, n_q, Hq, Hkv, D, cap = 2, 1, 2, 1, 8, 16
    q = synth.queries(B, n_q, Hq, D, 4)
    k, v = synth.kv_cache(B, cap, Hkv, D, [cap, cap], 5)
    o, l = oracle.attn(q, k, v, np.array([-4, cap + 9], np.int32), 0.3)
    o2, l2 = oracle.attn(q, k, v, np.array([0, cap], np.int32), 0.3)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(l[0]))


def test_gather_equals_masked_over_same_cells():
    B, n_q, Hq, Hkv, D, n_kv = 1, 2, 8, 2, 16, 300
    q = synth.queries(B, n_q, Hq, D, 6)
    k, v = synth.kv_cache(B, n_kv, Hkv, D, [n_kv], 6)
    idx = synth.topk_lists(B, n_q, Hkv, n_kv, 40, 8, seed=6)
    mask = synth.mask_from_lists(idx, n_kv)
    lens = np.array([n_kv], dtype=np.int32)
    for causal in (False, True):
        og, lg = oracle.attn(q, k, v, lens, 0.25, causal, idx=idx)
        om, lm = oracle.attn(q, k, v, lens, 0.25, causal, keep_mask=mask)
        assert pins.max_dev(og, om) <= pins.TOL and pins.max_dev(lg, lm) <= pins.TOL


def test_causal_single_query_equals_plain():
    q, k, v, lens = pins.small_case(n_q=1, seed=8)
    o1, l1 = oracle.attn(q, k, v, lens, 0.3, True)
    o0, l0 = oracle.attn(q, k, v, lens, 0.3, False)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)


def test_thread_count_does_not_change_result():
    q, k, v, lens = pins.small_case(seed=9)
    o1, l1 = oracle.attn(q, k, v, lens, 0.3, True, nthreads=1)
    o8, l8 = oracle.attn(q, k, v, lens, 0.3, True, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(l1, l8)


def test_rejects_bad_arguments():
    q, k, v, lens = pins.small_case(seed=10)
    with pytest.raises(ValueError):
        oracle.attn(q, k[:, :, :, :8], v[:, :, :, :8], lens, 0.3)  # D mismatch
    bad_q = synth.queries(2, 3, 3, 16, 1)  # Hq = 3 is not a multiple of Hkv = 2
    with pytest.raises(RuntimeError):
        oracle.attn(bad_q, k, v, lens, 0.3)


# --------------------------------------------------------------- mutants ----

MUTANTS = {
    "dropped_scale": ("s[t] = J->scale * dot;", "s[t] = dot;"),
    "wrong_exp_sign": ("double e = exp(s[t] - m_c[c]);", "double e = exp(m_c[c] - s[t]);"),
    "causal_off_by_one": ("lim = L - J->n_q + i + 1;", "lim = L - J->n_q + i;"),
    "wrong_head_map": ("int g = h / G;", "int g = h % J->Hkv;"),
    "k_v_swapped": ("const uint16_t *krow = kv_row(J, J->k, J->k_step, b, g, vis[t]);",
                    "const uint16_t *krow = kv_row(J, J->v, J->v_step, b, g, vis[t]);"),
    "q8_scale_step": ("*scale = amax / 127.0f;", "*scale = amax / 128.0f;"),
    "q8_truncating_round": ("float c = nearbyintf(", "float c = truncf("),
    "q8_page_row_swapped": ("size_t row = ((size_t)pg * J->Hkv + g) * J->page + (size_t)(j % J->page);",
                            "size_t row = ((size_t)pg * J->Hkv + g) * J->page + (size_t)(j / J->page);"),
    "q8_token_major_page": ("size_t row = ((size_t)pg * J->Hkv + g) * J->page + (size_t)(j % J->page);",
                            "size_t row = ((size_t)pg * J->page + (size_t)(j % J->page)) * J->Hkv + g;"),
    "q8_append_position": ("long long pos = s0 + t;", "long long pos = s0 + t + 1;"),
    "step_rows_off_by_one": ("for (int t = 0; t <= i; ++t) vis[n++]", "for (int t = 0; t < i; ++t) vis[n++]"),
    "step_rows_read_from_cache": (
        "return step + (((size_t)b * J->n_q + (size_t)(e - J->cap)) * J->Hkv + g) * (size_t)J->D;",
        "return cache + (((size_t)b * J->cap + (size_t)(e - J->cap)) * J->Hkv + g) * (size_t)J->D;"),
    "mask_ignored": ("if (J->keep_mask[mo] == 0) continue;", "(void)mo;"),
    "gather_limit_inclusive": ("if (j >= 0 && j < lim) vis[n++]", "if (j >= 0 && j <= lim) vis[n++]"),
    "lse_missing_max": ("if (lse) *lse = M + log(den);", "if (lse) *lse = log(den);"),
    "merge_without_rescale": ("double w = exp(m_c[c] - M);", "double w = 1.0;"),
    "query_index_transposed": (
        "size_t qo = (((size_t)b * J->n_q + i) * J->Hq + h) * (size_t)D;\n    double *o = J->out + qo;",
        "size_t qo = (((size_t)b * J->n_q + i) * J->Hq + h) * (size_t)D;\n    double *o = J->out + qo;\n"
        "    qo = (((size_t)b * J->Hq + h) * J->n_q + i) * (size_t)D;"),
    "clamp_missing": ("if (L > J->cap) L = J->cap;", ""),
    "topk_ties_highest_cell_first": ("return (x->j > y->j) - (x->j < y->j);",
                                     "return (x->j < y->j) - (x->j > y->j);"),
    "topk_nan_ranks_high": ("if (isnan(v)) v = -INFINITY;", "if (isnan(v)) v = INFINITY;"),
    "topk_tail_among_candidates": ("int n = lim - tail;", "int n = lim;"),
    "topk_one_short": ("int m = n < k ? n : k;", "int m = n < k ? n : k - 1;"),
    "topk_unsorted_lists": ("qsort(sel, (size_t)m, sizeof(int32_t), by_cell);", ""),
    "topk_smallest_first": ("if (x->v > y->v) return -1;", "if (x->v < y->v) return -1;"),
    "topk_causal_off_by_one": ("                lim = L - n_q + i + 1;", "                lim = L - n_q + i;"),
}


def _check_fails(lib) -> bool:
    for fn in pins.ALL_CHECKS.values():
        try:
            if not fn(lib) <= pins.TOL:
                return True
        except Exception:
            return True
    # the clamp mutant only shows with kv_lens beyond capacity; a planted
    # read past cap would also be visible here
    q, k, v, lens = pins.small_case(seed=12)
    big = np.array([45, 5], dtype=np.int32)
    try:
        o, l = oracle.attn(q, k, v, big, 0.3, lib=lib)
        ro, rl = pins.sdpa_reference(q, k, v, big, np.float32(0.3), False)
        if pins.max_dev(o, ro) > pins.TOL or pins.max_dev(l, rl) > pins.TOL:
            return True
    except Exception:
        return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    """Each planted mistake must fail some pin.  The mutant runs in a child
    process: a mutant that reads out of bounds may crash, which also counts
    as caught."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"libmut_{name}.so")
    oracle.build(str(path), so)
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle, test_oracle; "
            "sys.exit(0 if test_oracle._check_fails(oracle.load(%r)) else 3)"
            % (here, os.path.dirname(here), so))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, timeout=300)
    assert r.returncode != 3, f"mutant {name} passed every pin"
    if r.returncode != 0:
        assert r.returncode < 0 or r.returncode > 3, r.stderr.decode()[-2000:]
