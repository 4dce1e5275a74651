"""GPU whole-layer streaming (moe_layer_stream_*): two HBM banks, one layer each,
filled from pinned host memory on a side stream while the previous layer
computes.

The pages stream the next layer's experts while the current one computes during
prefill ("Three mechanisms", pipelined expert streaming).  Streaming changes only
where the weights come from, so every layer's output must equal, bit for bit,
the same layer computed from weights that were resident all along; one streamed
layer is also checked against the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
from helpers import assert_close_bf16_output, dev, log, to_dev
from routed_expert_ffn_layer_amd import layer as L
from routed_expert_ffn_layer_amd import moe

pytestmark = pytest.mark.gpu

E, K, H, I, T = 8, 2, 512, 256, 96


def _layers(dtype, n, seed):
    return [synth.small_layer(dtype, T, H, I, E, K, seed, layer=l) for l in range(n)]


def _resident(lay):
    b = L.LayerBuffers(T, E, K, H, I, lay["dtype"])
    eb = lay["experts"].shape[1]
    L.forward(b, to_dev(lay["logits"]), to_dev(lay["x"]), to_dev(lay["experts"]), eb, L.identity_slots(E))
    torch.cuda.synchronize()
    return b.y.clone()


def _streamed(lays, host_of_layer):
    """Run every layer through the two-bank pipeline; host_of_layer[l] is the
    pinned host buffer layer l is streamed from."""
    n = len(lays)
    dtype = lays[0]["dtype"]
    eb = lays[0]["experts"].shape[1]
    lb = E * eb
    banks = [torch.empty((E, eb), dtype=torch.uint8, device=dev()) for _ in range(2)]
    ptrs = (ctypes.c_void_p * n)(*[h.data_ptr() for h in host_of_layer])
    fill_stream = torch.cuda.Stream(device=dev())
    ls = moe.LayerStream(n, lb, banks[0], banks[1], fill_stream, host_layer_ptrs=ptrs)
    comp = torch.cuda.current_stream()
    b = L.LayerBuffers(T, E, K, H, I, dtype)
    ins = [(to_dev(l["logits"]), to_dev(l["x"])) for l in lays]
    slots = L.identity_slots(E)
    ys = []
    ls.fill(0, 0)
    for l in range(n):
        if l + 1 < n:
            ls.fill(l + 1, (l + 1) % 2)
        ls.acquire(l % 2, comp)
        L.forward(b, ins[l][0], ins[l][1], banks[l % 2], eb, slots)
        ys.append(b.y.clone())
        ls.release(l % 2, comp)
    torch.cuda.synchronize()
    ls.close()
    return ys


def _pinned(experts):
    t = torch.empty(experts.shape, dtype=torch.uint8, pin_memory=True)
    t.copy_(torch.from_numpy(np.ascontiguousarray(experts)))
    return t


@pytest.mark.parametrize("dtype", [synth.BF16, synth.MXFP4])
def test_streamed_layers_equal_resident(dtype, ora):
    log(f"layer stream: 5 layers dtype={dtype} T={T} H={H} I={I} E={E}")
    lays = _layers(dtype, 5, 4400 + dtype)
    host = [_pinned(l["experts"]) for l in lays]
    ys = _streamed(lays, host)
    for l, lay in enumerate(lays):
        assert torch.equal(ys[l], _resident(lay)), f"layer {l}"
    # one streamed layer against the oracle
    lay = lays[3]
    ref = ora.layer(dtype, lay["experts"], lay["x"], lay["logits"], K, H, I)
    r = assert_close_bf16_output(ys[3].float().cpu().numpy(), ref["y"], what="streamed layer 3 vs oracle")
    log(f"streamed layer 3: max err beyond the bf16 half-ulp / RMS = {r:.2e}")


def test_streamed_layers_aliased_host(ora):
    # six layers streamed from two host buffers (layer l reads host buffer l % 2):
    # each layer's output equals the resident layer built from the weights it read
    dtype = synth.BF16
    log("layer stream: 6 layers over 2 aliased host buffers")
    base = _layers(dtype, 2, 4500)
    host = [_pinned(l["experts"]) for l in base]
    lays = []
    for l in range(6):
        lay = synth.small_layer(dtype, T, H, I, E, K, 4501, layer=l)
        lay = dict(lay, experts=base[l % 2]["experts"])
        lays.append(lay)
    ys = _streamed(lays, [host[l % 2] for l in range(6)])
    for l, lay in enumerate(lays):
        assert torch.equal(ys[l], _resident(lay)), f"layer {l}"
