"""One MoE layer's routed-expert forward pass through the C ABI.

The caller supplies router logits, token activations and expert weights already
in HBM; this module only owns the per-shape buffers and calls the five library
entry points in order (route -> permute -> [cache lookup/fill] -> grouped FFN ->
combine).  With a cache, the FFN runs once per cache wave.
"""
import torch

from . import moe


class LayerBuffers:
    """Device buffers of one layer shape (T tokens, E experts, top-k, H, I)."""

    def __init__(self, T, E, k, H, I, wdt, I_shared=0, device="cuda"):
        self.T, self.E, self.k, self.H, self.I, self.wdt, self.I_shared = T, E, k, H, I, wdt, I_shared
        dev = torch.device(device)
        i32, f32 = torch.int32, torch.float32
        n = max(T * k, 1)
        self.topk_ids = torch.empty((T, k), dtype=i32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=f32, device=dev)
        self.counts = torch.empty(E, dtype=i32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=i32, device=dev)
        self.sorted_rows = torch.empty(n, dtype=i32, device=dev)
        self.inv_rows = torch.empty(n, dtype=i32, device=dev)
        self.out_rows = torch.empty((n, H), dtype=f32, device=dev)
        self.shared_out = torch.empty((max(T, 1), H), dtype=f32, device=dev) if I_shared else None
        ws = moe.moe_grouped_ffn_workspace(T, k, E, H, I, I_shared, wdt)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.ydt = moe.MOE_F32 if wdt == moe.MOE_F32 else moe.MOE_BF16
        self.y = torch.empty((T, H), dtype=f32 if self.ydt == moe.MOE_F32 else torch.bfloat16, device=dev)
        self.slot_table = torch.empty(E, dtype=i32, device=dev)
        self.slot_misses = torch.empty(E, dtype=i32, device=dev)
        self.addr_inplace = torch.empty(E, dtype=torch.int64, device=dev)


def identity_slots(E, device="cuda"):
    """Slot table of an all-resident layer: expert e lives in slot e."""
    return torch.arange(E, dtype=torch.int32, device=device)


def route(b: LayerBuffers, logits, stream=None):
    moe.moe_route(logits, b.k, b.topk_ids, b.topk_w, b.counts, b.offsets, b.sorted_rows, b.inv_rows, stream)


def ffn(b: LayerBuffers, x, slot_pool, slot_stride, slot_of_expert, shared_w=None, stream=None):
    moe.moe_grouped_ffn(b.wdt, slot_pool, slot_stride, slot_of_expert, shared_w, b.I_shared if shared_w is not None else 0,
                        x, b.offsets, b.sorted_rows, b.T, b.k, b.E, b.H, b.I, b.out_rows,
                        b.shared_out if shared_w is not None else None, b.workspace, stream)


def combine(b: LayerBuffers, with_shared, stream=None):
    moe.moe_combine(b.out_rows, b.topk_w, b.inv_rows, b.shared_out if with_shared else None, b.y, b.ydt, stream)


def forward(b: LayerBuffers, logits, x, slot_pool, slot_stride, slot_of_expert, shared_w=None, stream=None):
    """All experts resident at fixed slots (slot_of_expert on the device)."""
    route(b, logits, stream)
    ffn(b, x, slot_pool, slot_stride, slot_of_expert, shared_w, stream)
    combine(b, shared_w is not None, stream)
    return b.y


def forward_cached(b: LayerBuffers, cache: moe.MoeCache, layer, logits, x, slot_pool, slot_stride, shared_w=None,
                   stream=None):
    """Experts come from the global-LRU slot cache; one FFN pass per cache wave."""
    route(b, logits, stream)
    stats = cache.lookup_fill(layer, b.counts, 0, b.slot_table, stream)
    ffn(b, x, slot_pool, slot_stride, b.slot_table, shared_w, stream)
    waves = [stats]
    for w in range(1, stats["n_waves"]):
        waves.append(cache.lookup_fill(layer, None, w, b.slot_table, stream))
        ffn(b, x, slot_pool, slot_stride, b.slot_table, None, stream)
    combine(b, shared_w is not None, stream)
    return b.y, waves


def forward_cached_split(b: LayerBuffers, cache: moe.MoeCache, layer, logits, x, slot_pool, slot_stride,
                         shared_w=None, stream=None):
    """As forward_cached, but each wave's resident experts are computed while its
    misses are filled; the misses' FFN follows once their fills have landed."""
    route(b, logits, stream)
    waves = []
    w = 0
    while True:
        stats = cache.lookup_fill_split(layer, b.counts if w == 0 else None, w, b.slot_table, b.slot_misses, stream)
        waves.append(stats)
        ffn(b, x, slot_pool, slot_stride, b.slot_table, shared_w if w == 0 else None, stream)
        cache.wait_fills(stream)
        if stats["fill_bytes"]:
            ffn(b, x, slot_pool, slot_stride, b.slot_misses, None, stream)
        w += 1
        if w >= stats["n_waves"]:
            break
    combine(b, shared_w is not None, stream)
    return b.y, waves


def forward_cached_inplace(b: LayerBuffers, cache: moe.MoeCache, layer, logits, x, slot_pool, slot_stride,
                           shared_w=None, stream=None):
    """As forward_cached_split, with the cache's miss split: the step's in-place
    experts are computed straight from their pinned host copies (read by the GPU
    over the host link, no slot taken) right after the hits, while the filled
    misses are still on their way; the three FFN calls write disjoint rows and the
    combine adds them in the fixed order, so y equals the all-filled layer bit for
    bit."""
    route(b, logits, stream)
    waves = []
    w = 0
    while True:
        stats = cache.lookup_fill_inplace(layer, b.counts if w == 0 else None, w, b.slot_table, b.slot_misses,
                                          b.addr_inplace, stream)
        waves.append(stats)
        ffn(b, x, slot_pool, slot_stride, b.slot_table, shared_w if w == 0 else None, stream)
        if w == 0 and stats["inplace"]:
            moe.moe_grouped_ffn_addr(b.wdt, b.addr_inplace, None, 0, x, b.offsets, b.sorted_rows, b.T, b.k, b.E,
                                     b.H, b.I, b.out_rows, None, b.workspace, stream)
        cache.wait_fills(stream)
        if stats["fill_bytes"]:
            ffn(b, x, slot_pool, slot_stride, b.slot_misses, None, stream)
        w += 1
        if w >= max(stats["n_waves"], 1):
            break
    combine(b, shared_w is not None, stream)
    return b.y, waves
