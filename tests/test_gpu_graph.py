"""Resident MoE layers captured in a HIP graph and replayed.

A decode step over all-resident experts has no host synchronisation, so its
launches can be captured once and replayed (the bench does so).  Every replay
must equal the eager layer on the same inputs bit for bit, with eager work and
synchronisations between replays and new inputs copied into the captured
buffers before each replay.
"""
import numpy as np
import pytest
import torch

import synth
from helpers import dev, log, to_dev
from routed_expert_ffn_layer_amd import layer as L

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,T,H,I,E,k,shared", [
    (synth.BF16, 4, 512, 256, 16, 4, True),
    (synth.MXFP4, 8, 512, 256, 16, 3, False),   # token rows staged in LDS
    (synth.MXFP4, 1, 256, 128, 8, 2, False),
], ids=["bf16_T4_shared", "mxfp4_T8", "mxfp4_T1"])
def test_graph_replays_equal_eager(dtype, T, H, I, E, k, shared):
    log(f"graph replay dtype={dtype} T={T} H={H} I={I} E={E} k={k} shared={shared}")
    I_sh = 64 if shared else 0
    lays = [synth.small_layer(dtype, T, H, I, E, k, seed=610 + i, shared=shared, I_shared=I_sh) for i in range(4)]
    pool = to_dev(lays[0]["experts"])
    eb = lays[0]["experts"].shape[1]
    sh = to_dev(lays[0]["shared"]) if shared else None
    slots = L.identity_slots(E)

    def eager(lay):
        b = L.LayerBuffers(T, E, k, H, I, dtype, I_shared=I_sh)
        L.forward(b, to_dev(lay["logits"]), to_dev(lay["x"]), pool, eb, slots, sh)
        torch.cuda.synchronize()
        return b.y.clone()

    refs = [eager(lay) for lay in lays]
    # static inputs and buffers of the captured layer
    lg_s = to_dev(lays[0]["logits"]).clone()
    x_s = to_dev(lays[0]["x"]).clone()
    bg = L.LayerBuffers(T, E, k, H, I, dtype, I_shared=I_sh)
    L.forward(bg, lg_s, x_s, pool, eb, slots, sh)  # load kernels before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.forward(bg, lg_s, x_s, pool, eb, slots, sh)
    for rep in range(3):
        i = (rep + 1) % len(lays)
        lg_s.copy_(to_dev(lays[i]["logits"]))
        x_s.copy_(to_dev(lays[i]["x"]))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bg.y.view(torch.int16) if bg.y.dtype == torch.bfloat16 else bg.y,
                           refs[i].view(torch.int16) if refs[i].dtype == torch.bfloat16 else refs[i]), rep
        # eager work between replays
        again = eager(lays[(i + 1) % len(lays)])
        assert torch.equal(again, refs[(i + 1) % len(lays)])
