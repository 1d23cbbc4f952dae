"""A CPU model of the in-launch split merge, run over adversarial schedules.

The kernel's merge (decode_kernel in ck_decode_attn.hip) is a small protocol
between the workgroups of one unit (one sequence, KV head and row group),
and its correctness rests on orderings that a GPU test reaches only by
chance.  This file restates it step by step over a model memory and runs it
under random interleavings, with stores that land late and in any order,
and with few workgroups resident at once (a workgroup starts only when a
resident one has ended), over consecutive launches with changing lengths:

  * a split reads the unit's parity word, works out how many splits the
    length makes active (the rest leave at once), and counts itself started
    in the counter set the parity names;
  * it stores its partial, waits until those stores have landed, and takes
    its arrival rank with one atomic;
  * the last arrival clears the other counter set and flips the parity, then
    merges slice 0 (every partial has landed: each split waited for its own
    stores before arriving), claims every slice no helper took and merges
    those;
  * the arrival n-1-c may help with slice c: only if it saw every split
    started, by winning the slice's claim flag; it then waits (bounded) for
    the last arrival and merges; a helper that gives up sets the status bit
    and writes NaN over its slice.

Checked after every launch: every output written exactly once with the
merged value of this launch's partials, no wait that cannot end (it would
run into the poll limit and show as the status bit), and the next counter
set zero.  Planted mistakes in this model (a helper that ignores whether
every split started, no wait for the stores before arriving, no clearing of
the next set) make these checks fail.
"""
from __future__ import annotations

import math
import random

import pytest

NAN = float("nan")


class Memory:
    """Device memory at the point of coherence.  Plain stores land later
    (each is an event the scheduler applies at a time it picks); atomics act
    at once."""

    def __init__(self):
        self.v = {}
        self.pending = []  # (owner, address, value)

    def load(self, a):
        return self.v.get(a, 0)

    def store(self, owner, a, x):
        self.pending.append((owner, a, x))

    def atomic_add(self, a, x):
        old = self.load(a)
        self.v[a] = old + x
        return old

    def atomic_exch(self, a, x):
        old = self.load(a)
        self.v[a] = x
        return old

    def landed(self, owner):
        return not any(o == owner for o, _, _ in self.pending)

    def land_one(self, rng):
        _, a, x = self.pending.pop(rng.randrange(len(self.pending)))
        self.v[a] = x

    def drain(self):
        for _, a, x in self.pending:
            self.v[a] = x
        self.pending.clear()


PARITY = ("parity",)
STATUS = ("status",)


def started(par):
    return ("started", par)


def arrived(par):
    return ("arrived", par)


def flag(par, c):
    return ("flag", par, c)


def part(s, r, col):
    return ("acc", s, r, col)


def ml(s, r):
    return ("ml", s, r)


def slice_cols(c, ns, cols):
    return range(c * cols // ns, (c + 1) * cols // ns)


def merge(mem, c, ns, n_active, rows, cols, out):
    """Merge column slice c from the published partials (reads memory)."""
    for r in range(rows):
        ms = [mem.load(ml(s2, r)) for s2 in range(n_active)]
        ms = [x if isinstance(x, tuple) else (NAN, NAN) for x in ms]  # never written: garbage
        M = max(m for m, _ in ms)
        mu = 0.0 if M == -math.inf else M
        w = [2.0 ** (m - mu) for m, _ in ms]
        den = sum(wi * l for wi, (_, l) in zip(w, ms))
        for col in slice_cols(c, ns, cols):
            num = sum(wi * mem.load(part(s2, r, col)) for s2, wi in enumerate(w))
            out.setdefault((r, col), []).append(num / den if den > 0 else 0.0)


def workgroup(mem, s, n_active, n_slices, rows, cols, values, out, spin_limit, log, mistake=None):
    """Generator: split s of the unit; every yield is a point where other
    workgroups may run and stores may land."""
    par = mem.load(PARITY) & 1
    yield
    if s >= n_active:
        return
    if n_active == 1:  # a lone split writes the output itself
        for r in range(rows):
            m, l, acc = values[s][r]
            for col in range(cols):
                out.setdefault((r, col), []).append(acc[col] / l if l > 0 else 0.0)
        return
    mem.atomic_add(started(par), 1)
    yield
    seen = mem.load(started(par))            # read after its first tile
    yield
    for r in range(rows):
        m, l, acc = values[s][r]
        for col in range(cols):
            mem.store(s, part(s, r, col), acc[col])
        mem.store(s, ml(s, r), (m, l))
    yield
    while mistake != "no store wait" and not mem.landed(s):  # wait for its own stores
        yield
    rank = mem.atomic_add(arrived(par), 1)
    yield
    ns = min(n_slices, n_active)
    last = rank == n_active - 1
    helper = not last and rank >= n_active - ns
    if last:
        other = par ^ 1
        if mistake != "no clear":
            for c in range(n_slices):
                mem.store(s, flag(other, c), 0)
            mem.store(s, started(other), 0)
            mem.store(s, arrived(other), 0)
        mem.store(s, PARITY, other)
        merge(mem, 0, ns, n_active, rows, cols, out)
        log.append(("merged", s, 0))
        yield
        owned = [c for c in range(1, ns) if mem.atomic_exch(flag(par, c), 1) == 0]
        for c in owned:
            yield
            merge(mem, c, ns, n_active, rows, cols, out)
            log.append(("merged", s, c))
    elif helper:
        c = n_active - 1 - rank
        if (seen == n_active or mistake == "ignore started") and mem.atomic_exch(flag(par, c), 1) == 0:
            spins = 0
            while mem.load(arrived(par)) < n_active:
                spins += 1
                if spins > spin_limit:
                    mem.v[STATUS] = mem.load(STATUS) | 1
                    for r in range(rows):
                        for col in slice_cols(c, ns, cols):
                            out.setdefault((r, col), []).append(NAN)
                    log.append(("gave up", s, c))
                    return
                yield "wait"
            merge(mem, c, ns, n_active, rows, cols, out)
            log.append(("merged", s, c))


def run_launch(mem, S, n_active, n_slices, rows, cols, resident, rng, spin_limit=10_000, mistake=None):
    """One launch of S workgroups (the grid's splits), dispatched in order
    with at most `resident` running at once.  Returns (outputs by (row,
    column), expected, log)."""
    values = []
    for s in range(S):
        per_row = []
        for r in range(rows):
            m = rng.choice([-math.inf, rng.uniform(-4, 4), rng.uniform(-4, 4)])
            l = 0.0 if m == -math.inf else rng.uniform(0.5, 3.0)
            acc = [0.0 if m == -math.inf else rng.uniform(-2, 2) for _ in range(cols)]
            per_row.append((m, l, acc))
        values.append(per_row)
    out, log = {}, []
    queue = list(range(S))
    running = {}
    while queue or running or mem.pending:
        while queue and len(running) < resident:
            s = queue.pop(0)
            running[s] = workgroup(mem, s, n_active, n_slices, rows, cols, values, out, spin_limit, log, mistake)
        choices = list(running) + (["land"] if mem.pending else [])
        pick = rng.choice(choices)
        if pick == "land":
            mem.land_one(rng)
            continue
        try:
            next(running[pick])
        except StopIteration:
            del running[pick]
    mem.drain()
    expect = {}
    for r in range(rows):
        M = max(values[s][r][0] for s in range(n_active))
        mu = 0.0 if M == -math.inf else M
        w = [2.0 ** (values[s][r][0] - mu) for s in range(n_active)]
        den = sum(wi * values[s][r][1] for s, wi in enumerate(w))
        for col in range(cols):
            num = sum(wi * values[s][r][2][col] for s, wi in enumerate(w))
            expect[(r, col)] = num / den if den > 0 else 0.0
    return out, expect, log


def close(got, want):
    return abs(got - want) <= 1e-12 * (1 + abs(want))


def next_set_clear(mem, n_slices):
    par = mem.load(PARITY) & 1
    return (mem.load(started(par)) == 0 and mem.load(arrived(par)) == 0
            and all(mem.load(flag(par, c)) == 0 for c in range(n_slices)))


@pytest.mark.parametrize("S,rows,cols,slices,resident", [
    (2, 1, 4, 2, 2), (5, 2, 6, 3, 5), (8, 1, 8, 4, 8), (8, 2, 8, 4, 3), (8, 1, 8, 4, 1),
    (7, 1, 5, 5, 7), (6, 3, 12, 4, 2), (16, 2, 8, 8, 6)])
def test_every_slice_merged_once_over_random_schedules(S, rows, cols, slices, resident):
    rng = random.Random(1000 * S + 100 * rows + 10 * cols + resident)
    mem = Memory()
    keys = [(r, col) for r in range(rows) for col in range(cols)]
    for launch in range(120):
        n_active = max(1, min(S, rng.choice([1, 2, S, S, S - 1, rng.randint(1, S)])))
        out, expect, log = run_launch(mem, S, n_active, slices, rows, cols, resident, rng)
        assert sorted(out) == keys, (launch, log)
        for key in keys:
            assert len(out[key]) == 1, f"{key} written {len(out[key])} times: {log}"
            assert close(out[key][0], expect[key]), (launch, key, out[key][0], expect[key], log)
        assert mem.load(STATUS) == 0, log
        assert next_set_clear(mem, slices)


def test_one_resident_workgroup_never_waits_on_an_unscheduled_one():
    """With one workgroup resident at a time no helper may commit to a wait
    (it would wait for workgroups that cannot start, until the poll limit):
    the last arrival merges every slice alone."""
    rng = random.Random(7)
    mem = Memory()
    for _ in range(40):
        out, expect, log = run_launch(mem, 6, 6, 3, 2, 6, 1, rng)
        assert {s for kind, s, _ in log if kind == "merged"} == {5}
        assert all(len(v) == 1 and close(v[0], expect[k]) for k, v in out.items())
        assert mem.load(STATUS) == 0
        assert next_set_clear(mem, 3)


def test_tiny_poll_limit_gives_up_visibly():
    """With a poll limit of zero a helper that has to wait gives up: the
    status bit is set and its slice reads NaN; every workgroup still ends,
    and the last arrival still merges its own slices."""
    rng = random.Random(11)
    seen_fail = False
    for _ in range(200):
        mem = Memory()
        out, expect, log = run_launch(mem, 8, 8, 4, 2, 8, 8, rng, spin_limit=0)
        assert sorted(out) == sorted(expect)
        if mem.load(STATUS) & 1:
            seen_fail = True
            assert any(math.isnan(v[0]) for v in out.values())
            assert all(close(v[0], expect[k]) for k, v in out.items() if not math.isnan(v[0]))
        else:
            assert all(close(v[0], expect[k]) for k, v in out.items())
    assert seen_fail


def launch_is_right(mem, out, expect, slices):
    if sorted(out) != sorted(expect):
        return False
    if any(len(v) != 1 or not close(v[0], expect[k]) for k, v in out.items()):
        return False
    return mem.load(STATUS) == 0 and next_set_clear(mem, slices)


@pytest.mark.parametrize("mistake", ["ignore started", "no store wait", "no clear"])
def test_planted_mistakes_are_caught(mistake):
    """Each planted mistake makes some schedule produce a wrong output, a
    wait that runs into the poll limit, or a counter set left dirty: a helper
    that commits to waiting without having seen every split started, an
    arrival before the split's stores have landed, a last arrival that does
    not clear the next counter set."""
    rng = random.Random(sum(map(ord, mistake)))
    caught = False
    for trial in range(300):
        mem = Memory()
        S, slices = 8, 4
        resident = rng.choice([1, 2, 8])
        for _ in range(3):
            n_active = rng.choice([S, S - 1, 5])
            out, expect, log = run_launch(mem, S, n_active, slices, 2, 8, resident, rng, spin_limit=50,
                                          mistake=mistake)
            if not launch_is_right(mem, out, expect, slices):
                caught = True
                break
        if caught:
            break
    assert caught, mistake
