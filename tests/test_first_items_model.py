"""A model of the conv pair's first-item claims (CPU): eight per-XCD counters
hand out the launch's first producer items, a shared counter the rest, and
the workgroup that draws shared value P runs whatever the per-XCD counters
still hold before its own item.  The model steps workgroups in random order,
some of them never scheduled at all, and checks that every item completes
(no consumer waits forever) and runs exactly once.  Dependencies are the
conv pair's own halo ranges (chain_conv_dep_range)."""

import random

import pytest

import tile_level_sync_amd as tls

Q = 8  # per-XCD counters


def _deps(N, side, bm, C):
    deps = []
    for c in range(C):
        lo, hi = tls.chain_conv_dep_range(c, N, side, side, bm)
        deps.append(range(lo, hi + 1))
    return deps


def _simulate(P, C, deps, G, xcd_of, dead, rng, serial=False):
    """Runs the claim protocol; returns the run count of every item."""
    done = [0] * (P + C)
    runs = [0] * (P + C)
    nfirst = min(G, P)
    chunk = [max(0, (nfirst - x + Q - 1) // Q) for x in range(Q)]
    qnext = [0] * Q
    shared = [nfirst]
    end = P if serial else P + C
    state = {}  # wg -> list of pending items (front is current), or "exit"

    def take_first(x):
        i = qnext[x]
        qnext[x] += 1
        return x + Q * i if i < chunk[x] else None

    def next_items(w, first):
        items = []
        if first:
            it = take_first(xcd_of[w])
            if it is not None:
                return [it]
        t = shared[0]
        shared[0] += 1
        if t == P:  # the sweep, before the drawn value's own item
            for x in range(Q):
                while True:
                    it = take_first(x)
                    if it is None:
                        break
                    items.append(it)
        if t < end:
            items.append(t)
        return items

    live = [w for w in range(G) if w not in dead]
    for w in live:
        state[w] = ("first", [])
    steps = 0
    while live:
        steps += 1
        assert steps < 100000, "no progress"
        w = rng.choice(live)
        kind, items = state[w]
        if not items:
            items = next_items(w, kind == "first")
            if not items:
                live.remove(w)
                continue
            state[w] = ("run", items)
            continue
        it = items[0]
        if it >= P and not all(done[p] for p in deps[it - P]):
            # blocked: make sure some other live workgroup can progress
            if all(state[v][1] and state[v][1][0] >= P and
                   not all(done[p] for p in deps[state[v][1][0] - P]) for v in live):
                raise AssertionError("deadlock: every live workgroup waits")
            continue
        done[it] = 1
        runs[it] += 1
        state[w] = ("run", items[1:])
    return runs


@pytest.mark.parametrize("N,side,bm", [(2, 14, 64), (4, 28, 64), (1, 56, 128)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_every_item_runs_once_whoever_is_scheduled(N, side, bm, seed):
    rng = random.Random(seed * 100 + side)
    P = C = -(-N * side * side // bm)
    deps = _deps(N, side, bm, C)
    for G in (1, 3, 8, 13, P + C):
        xcd_of = [rng.randrange(Q) if seed else w % Q for w in range(G)]
        for frac_dead in (0.0, 0.3, 0.9):
            dead = set(w for w in range(G) if rng.random() < frac_dead)
            if len(dead) == G:
                dead.discard(0)
            runs = _simulate(P, C, deps, G, xcd_of, dead, rng)
            assert runs == [1] * (P + C), (G, frac_dead)


def test_serial_producer_launch_sweeps_at_its_end():
    """Under the serial policy the producer launch ends at P: the workgroup
    that draws P sweeps and then exits."""
    rng = random.Random(7)
    P = 20
    G = 12
    for dead_n in (0, 5, 11):
        dead = set(range(1, dead_n + 1))
        xcd_of = [w % Q for w in range(G)]
        runs = _simulate(P, 0, [], G, xcd_of, dead, rng, serial=True)
        assert runs == [1] * P
