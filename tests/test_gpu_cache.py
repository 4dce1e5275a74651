"""GPU expert-slot cache: fills from pinned host memory on a side stream.

The pages require expert output to stay bit-exact with no expert substitution
("Key Takeaways"), so a layer served through the cache, at any capacity and in
any number of waves, must equal the all-resident layer bit for bit; the cache
state after every step must equal the oracle's LRU state exactly.
"""
import numpy as np
import pytest
import torch

import synth
from helpers import dev, log, to_dev
from routed_expert_ffn_layer_amd import layer as L
from routed_expert_ffn_layer_amd import moe

pytestmark = pytest.mark.gpu


def _pinned_pool(experts_host):
    """[keys][expert_bytes] uint8 in pinned host memory."""
    t = torch.empty(experts_host.shape, dtype=torch.uint8, pin_memory=True)
    t.copy_(torch.from_numpy(np.ascontiguousarray(experts_host)))
    return t


def _device_cache(n_layers, E, S, eb, host_pool):
    stride = ((eb + 255) // 256) * 256
    slot_pool = torch.zeros((S, stride), dtype=torch.uint8, device=dev())
    fill_stream = torch.cuda.Stream(device=dev())
    c = moe.MoeCache(n_layers, E, S, expert_bytes=eb, slot_stride=stride, slot_pool=slot_pool,
                     host_pool=host_pool, fill_stream=fill_stream)
    return c, slot_pool, stride


def _resident_y(b, logits_d, x_d, pool_d, stride, E):
    L.forward(b, logits_d, x_d, pool_d, stride, L.identity_slots(E))
    torch.cuda.synchronize()
    return b.y.clone()


def _same_state(cache, lru):
    k1, t1 = cache.state()
    k2, t2 = lru.state()
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(t1, t2)


def test_tiny_layer_two_waves_and_single_token_steps(ora):
    cfg = synth.CONFIGS["tiny_f32"]
    lay = synth.tiny_layer()
    T, H, I, E, k, S = cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["k"], cfg["n_slots"]
    eb = synth.expert_bytes(synth.F32, H, I)
    host = _pinned_pool(lay["experts"])
    cache, slot_pool, stride = _device_cache(1, E, S, eb, host)
    lru = ora.LRU(S, 1, E)
    resident = to_dev(lay["experts"])
    x_d, lg_d = to_dev(lay["x"]), to_dev(lay["logits"])
    # (i) one 32-token step: 8 active experts through 4 slots -> 2 waves
    log("tiny cached: one 32-token step")
    b = L.LayerBuffers(T, E, k, H, I, synth.F32)
    y_ref = _resident_y(b, lg_d, x_d, resident, eb, E)
    b2 = L.LayerBuffers(T, E, k, H, I, synth.F32)
    y, waves = L.forward_cached(b2, cache, 0, lg_d, x_d, slot_pool, stride)
    torch.cuda.synchronize()
    assert waves[0]["n_waves"] == 2 and waves[0]["misses"] == 8
    assert torch.equal(y, y_ref)
    r = lru.step(0, b.counts.cpu().numpy())
    assert r["n_waves"] == 2
    _same_state(cache, lru)
    # (ii) 32 single-token steps
    log("tiny cached: 32 single-token steps")
    b1 = L.LayerBuffers(1, E, k, H, I, synth.F32)
    bc = L.LayerBuffers(1, E, k, H, I, synth.F32)
    misses = 0
    for t in range(T):
        y_ref = _resident_y(b1, lg_d[t:t + 1], x_d[t:t + 1], resident, eb, E)
        y, waves = L.forward_cached(bc, cache, 0, lg_d[t:t + 1], x_d[t:t + 1], slot_pool, stride)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), t
        r = lru.step(0, bc.counts.cpu().numpy())
        assert waves[0]["misses"] == int((r["hit"] == 0).sum())
        misses += waves[0]["misses"]
        _same_state(cache, lru)
    assert misses > 0
    cache.close()


@pytest.mark.parametrize("split", [False, True], ids=["whole", "split"])
def test_cached_trace_bitwise_equal_to_resident(ora, split):
    """Temporally correlated trace (reuse 0.7, Zipf 1.0) through a 37%-capacity
    cache over 6 layers, bf16 experts with a reduced hidden size; whole waves, or
    hits computed while the misses fill (split lookup)."""
    H, I, E, k, Ls, tokens = 256, 128, 64, 8, 6, 30
    S = int(0.37 * Ls * E)
    seed = 1005
    lg = synth.trace_logits(seed, tokens, Ls, E, s=1.0, reuse_p=0.7)
    experts = np.stack([synth.random_expert(synth.BF16, H, I, synth.rng(seed, 3, l, e)) for l in range(Ls)
                        for e in range(E)])
    eb = experts.shape[1]
    host = _pinned_pool(experts)
    cache, slot_pool, stride = _device_cache(Ls, E, S, eb, host)
    lru = ora.LRU(S, Ls, E)
    resident = to_dev(experts)
    b = L.LayerBuffers(1, E, k, H, I, synth.BF16)
    bc = L.LayerBuffers(1, E, k, H, I, synth.BF16)
    total = dict(accesses=0, misses=0)
    for t in range(tokens):
        x = to_dev(synth.encode_activations(synth.BF16, synth.normal_x(seed, 1, H, t)))
        for l in range(Ls):
            lg_d = to_dev(lg[t, l][None, :])
            y_ref = _resident_y(b, lg_d, x, resident[l * E:(l + 1) * E], eb, E)
            fwd = L.forward_cached_split if split else L.forward_cached
            y, waves = fwd(bc, cache, l, lg_d, x, slot_pool, stride)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (t, l)
            r = lru.step(l, bc.counts.cpu().numpy())
            assert waves[0]["misses"] == int((r["hit"] == 0).sum())
            total["accesses"] += waves[0]["accesses"]
            total["misses"] += waves[0]["misses"]
    _same_state(cache, lru)
    log(f"trace miss rate {total['misses'] / total['accesses']:.3f}")
    cache.close()


def test_split_lookup_waves_and_shared_expert(ora):
    """Split lookups over several waves (16 active experts, 6 slots) with a shared
    expert: every step equals the resident layer bit for bit and the cache state
    equals the oracle's LRU."""
    H, I, E, k, S, T = 128, 64, 16, 4, 6, 12
    lay = synth.small_layer(synth.BF16, T, H, I, E, k, seed=78, shared=True, I_shared=64)
    eb = lay["experts"].shape[1]
    host = _pinned_pool(lay["experts"])
    cache, slot_pool, stride = _device_cache(1, E, S, eb, host)
    lru = ora.LRU(S, 1, E)
    resident = to_dev(lay["experts"])
    shared = to_dev(lay["shared"])
    b = L.LayerBuffers(T, E, k, H, I, synth.BF16, I_shared=64)
    bc = L.LayerBuffers(T, E, k, H, I, synth.BF16, I_shared=64)
    for step in range(3):
        x_d = to_dev(synth.encode_activations(synth.BF16, synth.normal_x(78, T, H, step)))
        lg_d = to_dev(synth.normal_logits(78, T, E, step))
        L.forward(b, lg_d, x_d, resident, eb, L.identity_slots(E), shared)
        torch.cuda.synchronize()
        y_ref = b.y.clone()
        y, waves = L.forward_cached_split(bc, cache, 0, lg_d, x_d, slot_pool, stride, shared)
        torch.cuda.synchronize()
        assert waves[0]["n_waves"] >= 2
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), step
        r = lru.step(0, bc.counts.cpu().numpy())
        assert r["n_waves"] == waves[0]["n_waves"]
        _same_state(cache, lru)
    cache.close()


def test_device_fill_failure_keeps_cache_consistent(ora):
    """A fill failure forced from the host: the call fails with MOE_EHIP, no key
    points at a slot that may have been overwritten, and later steps are exact."""
    H, I, E, k, S = 128, 64, 16, 2, 6
    lay = synth.small_layer(synth.BF16, 4, H, I, E, k, seed=77)
    eb = lay["experts"].shape[1]
    host = _pinned_pool(lay["experts"])
    cache, slot_pool, stride = _device_cache(1, E, S, eb, host)
    resident = to_dev(lay["experts"])
    x_d, lg_d = to_dev(lay["x"]), to_dev(lay["logits"])
    b = L.LayerBuffers(4, E, k, H, I, synth.BF16)
    bc = L.LayerBuffers(4, E, k, H, I, synth.BF16)
    y_ref = _resident_y(b, lg_d, x_d, resident, eb, E)
    cache.inject_fill_failure(1)
    with pytest.raises(moe.MoeError) as e:
        L.forward_cached(bc, cache, 0, lg_d, x_d, slot_pool, stride)
    assert e.value.status == moe.MOE_EHIP
    torch.cuda.synchronize()
    keys, _ = cache.state()
    assert (keys >= 0).sum() == 0  # the cold cache only held the touched slots
    y, waves = L.forward_cached(bc, cache, 0, lg_d, x_d, slot_pool, stride)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    cache.close()


def test_device_resize_mid_trace(ora):
    """Elastic resize of a device cache between steps: shrink to a new pool, later
    grow to another; the kept experts are copied device to device (never from the
    host pool), every layer stays bitwise equal to the resident layer and the state
    equals the oracle's after every step."""
    H, I, E, k, Ls, tokens = 128, 64, 32, 4, 4, 24
    seed = 1009
    lg = synth.trace_logits(seed, tokens, Ls, E, s=1.0, reuse_p=0.7)
    experts = np.stack([synth.random_expert(synth.BF16, H, I, synth.rng(seed, 3, l, e)) for l in range(Ls)
                        for e in range(E)])
    eb = experts.shape[1]
    host = _pinned_pool(experts)
    S = 40
    cache, slot_pool, stride = _device_cache(Ls, E, S, eb, host)
    lru = ora.LRU(S, Ls, E)
    resident = to_dev(experts)
    b = L.LayerBuffers(1, E, k, H, I, synth.BF16)
    bc = L.LayerBuffers(1, E, k, H, I, synth.BF16)
    pool = slot_pool
    for t in range(tokens):
        if t in (8, 16):
            new_S = 11 if t == 8 else 60
            new_pool = torch.zeros((new_S, stride), dtype=torch.uint8, device=dev())
            log(f"resize to {new_S} at token {t}")
            moved = cache.resize(new_S, new_pool, stride)
            np.testing.assert_array_equal(moved, lru.resize(new_S))
            torch.cuda.synchronize()
            for s_new, s_old in enumerate(moved):   # the kept experts' bytes moved
                if s_old >= 0:
                    assert torch.equal(new_pool[s_new, :eb], pool[s_old, :eb])
            pool = new_pool
            _same_state(cache, lru)
        x = to_dev(synth.encode_activations(synth.BF16, synth.normal_x(seed, 1, H, t)))
        for l in range(Ls):
            lg_d = to_dev(lg[t, l][None, :])
            y_ref = _resident_y(b, lg_d, x, resident[l * E:(l + 1) * E], eb, E)
            y, waves = L.forward_cached(bc, cache, l, lg_d, x, pool, stride)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (t, l)
            lru.step(l, bc.counts.cpu().numpy())
            _same_state(cache, lru)
    cache.close()


@pytest.mark.parametrize("fill", [(1, 2), (0, 1), (2, 3)], ids=["half", "none", "two_thirds"])
def test_miss_split_bitwise_equal_to_resident(ora, fill):
    """The miss split: of each step's misses the first floor(m num/den + 1/2) are
    filled, the rest computed in place by the FFN reading their pinned host copies
    directly.  Every layer equals the all-resident layer bit for bit (the in-place
    rows merge through the same fixed-order combine), and the cache state equals
    the oracle's LRU with the same split after every step.  A shared expert and
    T = 3 tokens per step (several misses per step), bf16 experts."""
    H, I, E, k, Ls, tokens, T = 256, 128, 64, 8, 6, 16, 3
    S = int(0.37 * Ls * E)
    seed = 1105
    lg = synth.trace_logits(seed, tokens * T, Ls, E, s=1.0, reuse_p=0.7)
    experts = np.stack([synth.random_expert(synth.BF16, H, I, synth.rng(seed, 3, l, e)) for l in range(Ls)
                        for e in range(E)])
    shared = synth.random_expert(synth.BF16, H, 128, synth.rng(seed, 4))
    eb = experts.shape[1]
    host = _pinned_pool(experts)
    cache, slot_pool, stride = _device_cache(Ls, E, S, eb, host)
    cache.set_fill_fraction(*fill)
    lru = ora.LRU(S, Ls, E)
    resident = to_dev(experts)
    sh = to_dev(shared)
    b = L.LayerBuffers(T, E, k, H, I, synth.BF16, I_shared=128)
    bc = L.LayerBuffers(T, E, k, H, I, synth.BF16, I_shared=128)
    n_inplace = n_fills = 0
    for t in range(tokens):
        x = to_dev(synth.encode_activations(synth.BF16, synth.normal_x(seed, T, H, t)))
        for l in range(Ls):
            lg_d = to_dev(np.ascontiguousarray(lg[t * T:(t + 1) * T, l]))
            L.forward(b, lg_d, x, resident[l * E:(l + 1) * E], eb, L.identity_slots(E), sh)
            torch.cuda.synchronize()
            y_ref = b.y.clone()
            y, waves = L.forward_cached_inplace(bc, cache, l, lg_d, x, slot_pool, stride, sh)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (t, l)
            r = lru.step(l, bc.counts.cpu().numpy(), fill=fill)
            assert waves[0]["inplace"] == len(r["inplace"])
            assert waves[0]["misses"] == int((r["hit"] == 0).sum()) + len(r["inplace"])
            n_inplace += waves[0]["inplace"]
            n_fills += int((r["hit"] == 0).sum())
            _same_state(cache, lru)
    log(f"miss split {fill}: {n_fills} fills, {n_inplace} computed in place")
    assert n_inplace > 0
    assert (n_fills == 0) == (fill == (0, 1))
    cache.close()


@pytest.mark.parametrize("split", [False, True], ids=["whole", "split"])
def test_wide_wave_slot_tables(ora, split):
    """Waves that touch more experts than the slot-table kernel takes as arguments
    (240): 256 experts, 200 tokens of top-6 (about 253 experts active), 300 slots,
    so the first step's single wave fills about 250 experts and the slot tables go
    through the pinned staging ring; later steps (fewer active experts) through the
    argument kernel.  Bitwise against the all-resident layer, LRU state against the
    oracle after every step."""
    H, I, E, k, T, S = 128, 64, 256, 6, 200, 300
    seed = 4242
    experts = np.stack([synth.random_expert(synth.BF16, H, I, synth.rng(seed, 3, 0, e)) for e in range(E)])
    eb = experts.shape[1]
    host = _pinned_pool(experts)
    cache, slot_pool, stride = _device_cache(1, E, S, eb, host)
    lru = ora.LRU(S, 1, E)
    resident = to_dev(experts)
    wide = 0
    for step, n in enumerate((T, 3, T, 1)):
        x = to_dev(synth.encode_activations(synth.BF16, synth.normal_x(seed, n, H, step)))
        lg = to_dev(synth.normal_logits(seed, n, E, step))
        b = L.LayerBuffers(n, E, k, H, I, synth.BF16)
        bc = L.LayerBuffers(n, E, k, H, I, synth.BF16)
        y_ref = _resident_y(b, lg, x, resident, eb, E)
        fwd = L.forward_cached_split if split else L.forward_cached
        y, waves = fwd(bc, cache, 0, lg, x, slot_pool, stride)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), step
        active = int((bc.counts > 0).sum().item())
        wide += active > 240
        log(f"  step {step}: {n} tokens, {active} active experts, {waves[0]['misses']} misses")
        r = lru.step(0, bc.counts.cpu().numpy())
        assert waves[0]["misses"] == int((r["hit"] == 0).sum())
        _same_state(cache, lru)
    assert wide >= 1
    cache.close()
