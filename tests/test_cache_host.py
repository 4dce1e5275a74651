"""The library's cache policy (host-only handles) against the oracle's LRU, bit-exact:
access order, hit/miss, slot of every expert, fills, waves and final state; plus
failure handling forced from the host."""
import numpy as np
import pytest

import synth
from routed_expert_ffn_layer_amd import moe


def _counts(ids, E):
    return np.bincount(np.asarray(ids).ravel(), minlength=E).astype(np.int32)


def _step_both(lib_cache, ora_lru, layer, counts, E, S, fill=None):
    r = ora_lru.step(layer, counts, fill=fill)
    table, fills, st = lib_cache.lookup_host(layer, counts, 0)
    np.testing.assert_array_equal(lib_cache.step_inplace(), r["inplace"])
    assert st["inplace"] == len(r["inplace"])
    assert st["misses"] == int((r["hit"] == 0).sum()) + len(r["inplace"])
    assert st["n_waves"] == r["n_waves"]
    waves = [(table, fills, st)]
    for w in range(1, r["n_waves"]):
        waves.append(lib_cache.lookup_host(layer, None, w))
    for w, (table, fills, st) in enumerate(waves):
        sel = r["wave"] == w
        exp_table = np.full(E, -1, np.int32)
        exp_table[r["expert"][sel]] = r["slot"][sel]
        np.testing.assert_array_equal(table, exp_table)
        miss = sel & (r["hit"] == 0)
        assert fills == [(int(s), layer, int(e), w) for e, s in zip(r["expert"][miss], r["slot"][miss])]
        assert st["accesses"] == len(r["expert"]) + len(r["inplace"])
        assert st["hits"] == int(r["hit"].sum())
        assert st["cold_misses"] == int(((r["hit"] == 0) & (r["cold"] == 1)).sum()) + int(r["inplace_cold"].sum())
        assert st["wave_accesses"] == int(sel.sum())
    return r


def _same_state(lib_cache, ora_lru):
    k1, t1 = lib_cache.state()
    k2, t2 = ora_lru.state()
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(t1, t2)


@pytest.mark.parametrize("S", [1, 3, 8, 40, 200])
def test_random_steps_match_oracle(ora, S):
    g = np.random.default_rng(S)
    E, L = 24, 4
    c = moe.MoeCache(L, E, S)
    o = ora.LRU(S, L, E)
    for t in range(400):
        layer = int(g.integers(0, L))
        ids = g.choice(E, size=int(g.integers(0, 9)), replace=False)
        _step_both(c, o, layer, _counts(ids, E), E, S)
    _same_state(c, o)


def test_tiny_layer_waves_match_oracle(ora):
    # 8 experts, 4 slots: one 32-token step needs two waves; then 32 single-token steps
    cfg = synth.CONFIGS["tiny_f32"]
    L = synth.tiny_layer()
    ids, _, _ = ora.route_topk(L["logits"], cfg["k"])
    c = moe.MoeCache(1, cfg["E"], cfg["n_slots"])
    o = ora.LRU(cfg["n_slots"], 1, cfg["E"])
    r = _step_both(c, o, 0, _counts(ids, cfg["E"]), cfg["E"], cfg["n_slots"])
    assert r["n_waves"] == 2
    for t in range(cfg["T"]):
        _step_both(c, o, 0, _counts(ids[t], cfg["E"]), cfg["E"], cfg["n_slots"])
    _same_state(c, o)


def test_cached_trace_prefix_matches_oracle(ora):
    # the cached-trace recipe: 48 layers x 256 experts, top-8, 37% capacity; first 40 tokens
    cfg = synth.CONFIGS["cached_trace_bf16"]
    E, L, k, S = cfg["E"], cfg["layers"], cfg["k"], synth.cache_slots_for(cfg)
    lg = synth.trace_logits(cfg["seed"], 40, L, E, s=cfg["zipf_s"], reuse_p=cfg["reuse_p"])
    c = moe.MoeCache(L, E, S)
    o = ora.LRU(S, L, E)
    for t in range(40):
        for l in range(L):
            ids, _, _ = ora.route_topk(lg[t, l][None, :], k)
            _step_both(c, o, l, _counts(ids, E), E, S)
    _same_state(c, o)


def test_out_of_order_wave_is_rejected():
    c = moe.MoeCache(1, 8, 2)
    c.lookup_host(0, np.ones(8, np.int32), 0)      # 4 waves
    with pytest.raises(moe.MoeError) as e:
        c.lookup_host(0, None, 2)
    assert e.value.status == moe.MOE_ESTATE


def test_injected_fill_failure_invalidates_touched_slots_only(ora):
    E, S = 16, 6
    c = moe.MoeCache(1, E, S)
    g = np.random.default_rng(9)
    for t in range(30):
        c.lookup_host(0, _counts(g.choice(E, size=3, replace=False), E), 0)
    keys_before, ticks_before = c.state()
    counts = _counts([1, 2, 3, 4, 5], E)
    # the planned fills of this step, from a twin handle in the same state
    twin = moe.MoeCache(1, E, S)
    g = np.random.default_rng(9)
    for t in range(30):
        twin.lookup_host(0, _counts(g.choice(E, size=3, replace=False), E), 0)
    _, planned, _ = twin.lookup_host(0, counts, 0)
    assert len(planned) >= 2
    c.inject_fill_failure(1)  # the second fill fails
    with pytest.raises(moe.MoeError) as e:
        c.lookup_host(0, counts, 0)
    assert e.value.status == moe.MOE_EHIP
    keys_after, ticks_after = c.state()
    touched = {planned[0][0], planned[1][0]}
    for s in range(S):
        if s in touched:
            assert keys_after[s] == -1
        else:
            assert keys_after[s] == keys_before[s] and ticks_after[s] == ticks_before[s]
    # the handle keeps working: a fresh step succeeds and refills what it needs
    table, fills, st = c.lookup_host(0, counts, 0)
    assert all(table[e] >= 0 for e in (1, 2, 3, 4, 5))
    assert len(set(table[[1, 2, 3, 4, 5]])) == 5


def test_resize_between_steps_matches_oracle(ora):
    """Elastic resize of a host-only handle: same kept keys, slots and moves as the
    oracle; later steps identical; resizing inside an open step is refused."""
    g = np.random.default_rng(11)
    E, L, S = 16, 3, 12
    c = moe.MoeCache(L, E, S)
    o = ora.LRU(S, L, E)
    for t, new_S in ((60, 5), (120, 30), (150, 1), (170, 9)):
        while True:
            layer = int(g.integers(0, L))
            ids = g.choice(E, size=int(g.integers(1, 7)), replace=False)
            _step_both(c, o, layer, _counts(ids, E), E, c.n_slots)
            t -= 1
            if t <= 0:
                break
        np.testing.assert_array_equal(c.resize(new_S), o.resize(new_S))
        _same_state(c, o)
    for _ in range(50):
        layer = int(g.integers(0, L))
        _step_both(c, o, layer, _counts(g.choice(E, size=4, replace=False), E), E, c.n_slots)
    _same_state(c, o)
    # a step with two waves left open: resize refused, the cache untouched
    c2 = moe.MoeCache(1, E, 2)
    c2.lookup_host(0, _counts(np.arange(5), E), 0)
    with pytest.raises(moe.MoeError) as e:
        c2.resize(4)
    assert e.value.status == moe.MOE_ESTATE
    with pytest.raises(moe.MoeError):
        c.resize(0)


def _ordered_dict_lru_misses(steps, S):
    """Independent LRU (collections.OrderedDict, most recent last) over the same
    access order: per step the hits ascending, then the misses ascending, hit or
    miss judged before the step.  Returns (misses, resident keys oldest first)."""
    from collections import OrderedDict
    lru = OrderedDict()
    misses = 0
    for keys in steps:
        hits = sorted(k for k in keys if k in lru)
        miss = sorted(k for k in keys if k not in lru)
        for k in hits:
            lru.move_to_end(k)
        for k in miss:
            if len(lru) >= S:
                lru.popitem(last=False)
            lru[k] = True
        misses += len(miss)
    return misses, list(lru.keys())


def test_cached_trace_full_matches_oracle(ora):
    """The whole cached-trace workload: 1000 tokens x 48 layers x 256 experts, top-8,
    4546 slots (37% of the pool), cold start.  The library's host handle and the
    oracle make the same plan at every step (slots, fills, waves) and end in the
    same state; their miss count equals an OrderedDict LRU's, and the cache runs
    full and evicts (the first eviction comes after about 90 tokens)."""
    cfg = synth.CONFIGS["cached_trace_bf16"]
    E, L, k, S, n_tok = cfg["E"], cfg["layers"], cfg["k"], synth.cache_slots_for(cfg), cfg["tokens"]
    assert S == 4546
    lg = synth.trace_logits(cfg["seed"], n_tok, L, E, s=cfg["zipf_s"], reuse_p=cfg["reuse_p"])
    ids, _, _ = ora.route_topk(lg.reshape(-1, E), k)
    ids = ids.reshape(n_tok, L, k)
    c = moe.MoeCache(L, E, S)
    o = ora.LRU(S, L, E)
    misses = accesses = 0
    first_evict = None
    steps = []
    for t in range(n_tok):
        for l in range(L):
            counts = _counts(ids[t, l], E)
            r = _step_both(c, o, l, counts, E, S)
            accesses += len(r["expert"])
            misses += int((r["hit"] == 0).sum())
            if first_evict is None and misses > S:
                first_evict = t
            steps.append([l * E + int(e) for e in np.flatnonzero(counts)])
    _same_state(c, o)
    ref_misses, ref_keys = _ordered_dict_lru_misses(steps, S)
    assert misses == ref_misses
    keys, ticks = c.state()
    order = [int(kk) for kk, _ in sorted((kk, tt) for kk, tt in zip(keys, ticks) if kk >= 0)]
    assert sorted(order) == sorted(ref_keys)
    by_tick = [int(kk) for tt, kk in sorted((tt, kk) for kk, tt in zip(keys, ticks) if kk >= 0)]
    assert by_tick == ref_keys
    assert accesses == n_tok * L * k
    assert first_evict is not None and first_evict < n_tok // 2
    print(f"cached trace: {misses} misses of {accesses} accesses ({misses / accesses:.2%}), "
          f"first eviction at token {first_evict}")


@pytest.mark.parametrize("fill", [(0, 1), (1, 2), (2, 3), (3, 4)])
def test_miss_split_matches_oracle(ora, fill):
    """The library's split of misses (filled / computed in place) against the
    oracle's: same slots, fills, in-place experts and final state, on the
    cached-trace recipe at reduced size and on random steps with several waves."""
    cfg = synth.CONFIGS["cached_trace_bf16"]
    E, L, k = cfg["E"], 6, cfg["k"]
    S = int(0.37 * L * E)
    lg = synth.trace_logits(cfg["seed"], 60, L, E, s=cfg["zipf_s"], reuse_p=cfg["reuse_p"])
    c = moe.MoeCache(L, E, S)
    c.set_fill_fraction(*fill)
    o = ora.LRU(S, L, E)
    n_inplace = 0
    for t in range(60):
        for l in range(L):
            ids, _, _ = ora.route_topk(lg[t, l][None, :], k)
            r = _step_both(c, o, l, _counts(ids, E), E, S, fill=fill)
            n_inplace += len(r["inplace"])
    _same_state(c, o)
    assert n_inplace > 0
    g = np.random.default_rng(3)
    E2, S2 = 24, 5
    c2 = moe.MoeCache(3, E2, S2)
    c2.set_fill_fraction(*fill)
    o2 = ora.LRU(S2, 3, E2)
    for t in range(200):
        layer = int(g.integers(0, 3))
        _step_both(c2, o2, layer, _counts(g.choice(E2, size=int(g.integers(0, 12)), replace=False), E2), E2, S2,
                   fill=fill)
    _same_state(c2, o2)


def test_fill_fraction_arguments():
    c = moe.MoeCache(1, 8, 2)
    for bad in ((-1, 2), (3, 2), (0, 0)):
        with pytest.raises(moe.MoeError) as e:
            c.set_fill_fraction(*bad)
        assert e.value.status == moe.MOE_EINVAL
    c.lookup_host(0, np.ones(8, np.int32), 0)      # a step of 4 waves left open
    with pytest.raises(moe.MoeError) as e:
        c.set_fill_fraction(1, 2)
    assert e.value.status == moe.MOE_ESTATE
