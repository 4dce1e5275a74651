"""Pins of the oracle's global LRU expert cache.

A brute-force list LRU (most recent at the end, O(n*S)) replays the same steps
from the stated access rule; closed-form miss counts and Belady's optimal
policy bound it from outside.
"""
import json
import math
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class BruteLRU:
    def __init__(self, S):
        self.S = S
        self.order = []          # resident keys, least recent first
        self.slot = {}           # key -> slot
        self.seen = set()

    def step(self, layer, E, counts, fill=None):
        """fill = (num, den): of the m misses only the first floor(m num / den + 1/2)
        are accessed; the others (self.inplace, with their cold flags) are not."""
        active = [e for e in range(E) if counts[e] > 0]
        resident = set(self.order)
        misses = [e for e in active if layer * E + e not in resident]
        self.inplace = []
        if fill is not None:
            from fractions import Fraction
            q = math.floor(Fraction(len(misses) * fill[0], fill[1]) + Fraction(1, 2))
            self.inplace = [(e, int(layer * E + e not in self.seen)) for e in misses[q:]]
            misses = misses[:q]
        seq = [e for e in active if layer * E + e in resident] + misses
        recs = []
        for a, e in enumerate(seq):
            key = layer * E + e
            cold = key not in self.seen
            self.seen.add(key)
            ev = -1
            if key in self.slot:
                hit = True
                self.order.remove(key)
            else:
                hit = False
                used = set(self.slot.values())
                free = [s for s in range(self.S) if s not in used]
                if free:
                    s = free[0]
                else:
                    ev = self.order.pop(0)
                    s = self.slot.pop(ev)
                self.slot[key] = s
            self.order.append(key)
            recs.append((e, int(hit), self.slot[key], a // self.S, int(cold), ev))
        return recs


def brute_resize(b, new_S):
    """Truncation written out: keep the new_S most recently used keys, most recent
    in slot 0; return the old slot of each new slot (-1 empty)."""
    kept = b.order[::-1][:new_S]                 # most recent first
    moved = [b.slot[k] for k in kept] + [-1] * (new_S - len(kept))
    b.order = [k for k in b.order if k in set(kept)]
    b.slot = {k: s for s, k in enumerate(kept)}
    b.S = new_S
    return moved


def _counts_from_ids(ids, E):
    return np.bincount(np.asarray(ids).ravel(), minlength=E).astype(np.int32)


def _run_both(ora, S, L, E, steps):
    o = ora.LRU(S, L, E)
    b = BruteLRU(S)
    for layer, counts in steps:
        r = o.step(layer, counts)
        recs = b.step(layer, E, counts)
        got = list(zip(r["expert"], r["hit"], r["slot"], r["wave"], r["cold"], r["evicted"]))
        assert [tuple(int(v) for v in g) for g in got] == recs
        assert r["n_waves"] == (0 if not recs else (len(recs) - 1) // S + 1)
    keys, ticks = o.state()
    # same resident set, same slots, same recency order
    res = {int(k): s for s, k in enumerate(keys) if k >= 0}
    assert res == b.slot
    by_tick = [int(keys[s]) for s in np.argsort(ticks) if keys[s] >= 0]
    assert by_tick == b.order
    return o, b


def test_lru_matches_brute_force_random_steps(ora):
    g = np.random.default_rng(0)
    E, L = 16, 3
    steps = []
    for t in range(300):
        layer = t % L
        ids = g.choice(E, size=g.integers(1, 6), replace=False)
        steps.append((layer, _counts_from_ids(ids, E)))
    for S in (1, 2, 5, 7, 16, 48, 100):
        _run_both(ora, S, L, E, steps)


def test_lru_zipf_trace_matches_brute_force(ora):
    # the cached-trace recipe at reduced size (60 tokens, 4 layers, 64 experts, top-8)
    E, L, k, S = 64, 4, 8, 60
    lg = synth.trace_logits(77, 60, L, E, s=1.0, reuse_p=0.7)
    steps = []
    for t in range(60):
        for l in range(L):
            ids, _, _ = ora.route_topk(lg[t, l][None, :], k)
            steps.append((l, _counts_from_ids(ids, E)))
    _run_both(ora, S, L, E, steps)


def test_capacity_at_least_distinct_keys_misses_only_cold(ora):
    g = np.random.default_rng(1)
    E, L = 12, 2
    o = ora.LRU(E * L, L, E)
    distinct, misses = set(), 0
    for t in range(200):
        layer = t % L
        ids = g.choice(E, size=3, replace=False)
        r = o.step(layer, _counts_from_ids(ids, E))
        misses += int((r["hit"] == 0).sum())
        distinct |= {layer * E + int(e) for e in ids}
    assert misses == len(distinct)


def test_single_slot_misses_equal_key_changes(ora):
    g = np.random.default_rng(2)
    E, L = 5, 2
    o = ora.LRU(1, L, E)
    prev, changes, misses = None, 0, 0
    for t in range(300):
        layer = int(g.integers(0, L))
        e = int(g.integers(0, E))
        key = layer * E + e
        changes += key != prev
        prev = key
        c = np.zeros(E, np.int32); c[e] = 1
        r = o.step(layer, c)
        misses += int(r["hit"][0] == 0)
        assert r["slot"][0] == 0
    assert misses == changes


def _belady_misses(seq, S):
    cache, misses = set(), 0
    for i, key in enumerate(seq):
        if key in cache:
            continue
        misses += 1
        if len(cache) >= S:
            def next_use(k):
                for j in range(i + 1, len(seq)):
                    if seq[j] == k:
                        return j
                return math.inf
            cache.remove(max(cache, key=next_use))
        cache.add(key)
    return misses


def test_lru_misses_at_least_belady(ora):
    g = np.random.default_rng(3)
    E = 10
    seq = [int(v) for v in g.zipf(1.4, size=400) % E]
    for S in (1, 2, 3, 5):
        o = ora.LRU(S, 1, E)
        misses = 0
        for e in seq:
            c = np.zeros(E, np.int32); c[e] = 1
            misses += int(o.step(0, c)["hit"][0] == 0)
        assert misses >= _belady_misses(seq, S)


def test_waves_when_active_set_exceeds_capacity(ora):
    # tiny layer: 8 experts active, 4 slots -> 2 waves; every wave's experts resident together
    E, S = 8, 4
    o = ora.LRU(S, 1, E)
    r = o.step(0, np.ones(E, np.int32))
    assert r["n_waves"] == 2
    assert list(r["wave"]) == [0, 0, 0, 0, 1, 1, 1, 1]
    for w in range(2):
        slots = r["slot"][r["wave"] == w]
        assert sorted(slots) == list(range(S))
    # second identical step: experts 4..7 resident (hits first), 0..3 missing
    r2 = o.step(0, np.ones(E, np.int32))
    assert list(r2["expert"]) == [4, 5, 6, 7, 0, 1, 2, 3]
    assert list(r2["hit"]) == [1, 1, 1, 1, 0, 0, 0, 0]


def test_hits_never_evicted_by_their_own_step(ora):
    g = np.random.default_rng(4)
    E, L, S = 32, 2, 10
    o = ora.LRU(S, L, E)
    for t in range(500):
        layer = t % L
        ids = g.choice(E, size=int(g.integers(1, S + 1)), replace=False)
        r = o.step(layer, _counts_from_ids(ids, E))
        own = {layer * E + int(e) for e in ids}
        assert not (set(int(v) for v in r["evicted"]) & own)
        keys, _ = o.state()
        assert own <= set(int(k) for k in keys)


def test_cached_trace_capacity_from_pages():
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    cfg = synth.CONFIGS["cached_trace_bf16"]
    assert cfg["capacity_frac"] == fig["cache_capacity_fraction"]["value"]
    assert synth.cache_slots_for(cfg) == 4546


def test_workload_shape_against_pages():
    """The MXFP4 layer shape reproduces the pages' pool-size and parameter figures."""
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    c = synth.CONFIGS["decode_mxfp4"]
    assert c["E"] == fig["routed_experts_per_layer"]["value"]
    assert c["k"] == fig["active_experts_per_token_per_layer"]["value"]
    assert c["layers"] == fig["moe_layers"]["value"]
    pool = c["layers"] * c["E"] * synth.expert_bytes(synth.MXFP4, c["H"], c["I"])
    assert abs(pool / 1e9 - fig["fp4_pool_gb_roughly"]["value"]) / fig["fp4_pool_gb_roughly"]["value"] < 0.1
    routed = c["layers"] * c["E"] * 3 * c["H"] * c["I"]
    assert routed < fig["total_params_billion"]["value"] * 1e9
    active_routed = c["layers"] * c["k"] * 3 * c["H"] * c["I"]
    assert active_routed < fig["active_params_billion"]["value"] * 1e9


def test_lru_resize_matches_brute_force_truncation(ora):
    """Elastic resize between steps (shrink, grow, down to one slot, beyond the key
    count): the oracle keeps the most recent keys, most recent first, and later
    steps go on exactly as the brute-force LRU after the same truncation."""
    g = np.random.default_rng(5)
    E, L = 12, 3
    o = ora.LRU(20, L, E)
    b = BruteLRU(20)
    schedule = {40: 7, 80: 30, 120: 1, 140: 16, 200: 50}
    for t in range(260):
        if t in schedule:
            moved = o.resize(schedule[t])
            assert list(moved) == brute_resize(b, schedule[t])
        layer = int(g.integers(L))
        ids = np.stack([g.choice(E, size=3, replace=False) for _ in range(int(g.integers(1, 4)))])
        counts = _counts_from_ids(ids, E)
        r = o.step(layer, counts)
        recs = b.step(layer, E, counts)
        got = list(zip(r["expert"], r["hit"], r["slot"], r["wave"], r["cold"], r["evicted"]))
        assert [tuple(int(v) for v in x) for x in got] == recs, t
    keys, ticks = o.state()
    assert {int(k): s for s, k in enumerate(keys) if k >= 0} == b.slot
    assert [int(keys[s]) for s in np.argsort(ticks) if keys[s] >= 0] == b.order


def test_lru_resize_closed_forms(ora):
    E = 8
    o = ora.LRU(6, 1, E)
    o.step(0, np.array([1, 1, 1, 1, 0, 0, 0, 0], np.int32))   # keys 0..3 in slots 0..3
    o.step(0, np.array([0, 0, 1, 0, 0, 0, 0, 0], np.int32))   # key 2 most recent
    keys_before, _ = o.state()
    moved = o.resize(1)                                       # only the most recent survives
    assert list(moved) == [int(np.where(keys_before == 2)[0][0])]
    keys, _ = o.state()
    assert list(keys) == [2]
    moved = o.resize(4)                                       # growing keeps everything
    assert list(moved) == [0, -1, -1, -1]
    r = o.step(0, np.array([0, 0, 1, 1, 0, 0, 0, 0], np.int32))
    assert list(r["hit"]) == [1, 0] and list(r["slot"]) == [0, 1]


# ---- the miss split: part of a step's misses computed in place, not accessed ----

def _run_split(ora, S, L, E, steps, fill):
    o = ora.LRU(S, L, E)
    b = BruteLRU(S)
    n_inplace = 0
    for layer, counts in steps:
        r = o.step(layer, counts, fill=fill)
        recs = b.step(layer, E, counts, fill=fill)
        got = list(zip(r["expert"], r["hit"], r["slot"], r["wave"], r["cold"], r["evicted"]))
        assert [tuple(int(v) for v in g) for g in got] == recs
        assert [(int(e), int(c)) for e, c in zip(r["inplace"], r["inplace_cold"])] == b.inplace
        n_inplace += len(b.inplace)
    keys, ticks = o.state()
    res = {int(k): s for s, k in enumerate(keys) if k >= 0}
    assert res == b.slot
    assert [int(keys[s]) for s in np.argsort(ticks) if keys[s] >= 0] == b.order
    return n_inplace


@pytest.mark.parametrize("fill", [(0, 1), (1, 3), (1, 2), (2, 3), (3, 4), (1, 1)])
def test_lru_split_matches_brute_force(ora, fill):
    g = np.random.default_rng(5)
    E, L = 16, 3
    steps = []
    for t in range(300):
        ids = g.choice(E, size=g.integers(1, 7), replace=False)
        steps.append((t % L, _counts_from_ids(ids, E)))
    for S in (1, 3, 8, 20):
        n = _run_split(ora, S, L, E, steps, fill)
        assert (n == 0) == (fill == (1, 1))


def test_lru_split_closed_forms(ora):
    E = 8
    # on an empty cache every active expert misses: the filled count follows the
    # rounding rule floor(m num / den + 1/2) (halves round up)
    for m, fill, q in ((1, (1, 2), 1), (3, (1, 2), 2), (1, (1, 3), 0), (2, (1, 3), 1), (5, (2, 5), 2),
                       (4, (0, 1), 0), (4, (1, 1), 4), (7, (3, 4), 5)):
        o = ora.LRU(4, 1, E)
        r = o.step(0, _counts_from_ids(np.arange(m), E), fill=fill)
        assert len(r["expert"]) == q and list(r["expert"]) == list(range(q))
        assert list(r["inplace"]) == list(range(q, m)) and all(r["inplace_cold"] == 1)
    # fill fraction 0: the cache never changes, every miss is computed in place
    o = ora.LRU(5, 2, E)
    g = np.random.default_rng(1)
    for t in range(50):
        r = o.step(t % 2, _counts_from_ids(g.choice(E, size=3, replace=False), E), fill=(0, 1))
        assert len(r["expert"]) == 0 and len(r["inplace"]) == 3
    keys, ticks = o.state()
    assert np.all(keys == -1) and np.all(ticks == -1)
    # fill fraction 1 is the unsplit step
    o1, o2 = ora.LRU(6, 2, E), ora.LRU(6, 2, E)
    for t in range(80):
        c = _counts_from_ids(g.choice(E, size=int(g.integers(1, 5)), replace=False), E)
        a, b = o1.step(t % 2, c), o2.step(t % 2, c, fill=(1, 1))
        for key in ("expert", "hit", "slot", "wave", "cold", "evicted"):
            assert np.array_equal(a[key], b[key])
        assert len(b["inplace"]) == 0
    assert all(np.array_equal(x, y) for x, y in zip(o1.state(), o2.state()))
    # in-place keys are not accessed: a key computed in place misses again next step
    # and is cold until it is filled once
    o = ora.LRU(4, 1, E)
    r = o.step(0, _counts_from_ids([2, 5], E), fill=(1, 2))
    assert list(r["expert"]) == [2] and list(r["inplace"]) == [5]
    r = o.step(0, _counts_from_ids([5], E), fill=(1, 1))
    assert list(r["hit"]) == [0] and list(r["cold"]) == [1]
