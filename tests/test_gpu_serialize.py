"""Serialized against asynchronous execution, bit for bit.

A 37%-capacity cached trace (fills from pinned host memory on a side stream, fenced
by events against the FFN on the compute stream; whole and split lookups, so hits
are computed while misses fill) runs in a child process twice: once as usual and
once with the HIP runtime serializing every kernel launch and copy
(AMD_SERIALIZE_KERNEL=3, AMD_SERIALIZE_COPY=3).  A missing wait (the FFN reading a
slot before its fill lands, a fill overwriting a slot an earlier FFN still reads)
could change the asynchronous run's outputs, never the serialized one's; the two
runs' outputs and final cache states must be identical.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import hashlib, sys
ROOT = sys.argv[1]
sys.path.insert(0, ROOT)
import numpy as np
import torch
import synth
from routed_expert_ffn_layer_amd import layer as L
from routed_expert_ffn_layer_amd import moe

print("child: cached trace", flush=True)
dev = torch.device("cuda:0")
H, I, E, k, Ls, tokens = 256, 128, 64, 8, 6, 30
S = int(0.37 * Ls * E)
seed = 1005
lg = synth.trace_logits(seed, tokens, Ls, E, s=1.0, reuse_p=0.7)
experts = np.stack([synth.random_expert(synth.BF16, H, I, synth.rng(seed, 3, l, e)) for l in range(Ls)
                    for e in range(E)])
eb = experts.shape[1]
host = torch.empty(experts.shape, dtype=torch.uint8, pin_memory=True)
host.copy_(torch.from_numpy(np.ascontiguousarray(experts)))
stride = ((eb + 255) // 256) * 256
slot_pool = torch.zeros((S, stride), dtype=torch.uint8, device=dev)
fill_stream = torch.cuda.Stream(device=dev)
cache = moe.MoeCache(Ls, E, S, expert_bytes=eb, slot_stride=stride, slot_pool=slot_pool, host_pool=host,
                     fill_stream=fill_stream)
bc = L.LayerBuffers(1, E, k, H, I, synth.BF16)
xs = torch.from_numpy(np.stack([synth.encode_activations(synth.BF16, synth.normal_x(seed, 1, H, t))
                                for t in range(tokens)])).to(dev)
lgd = torch.from_numpy(np.ascontiguousarray(lg)).to(dev)
ys = []
for t in range(tokens):
    for l in range(Ls):
        fwd = L.forward_cached_split if l % 2 else L.forward_cached
        y, waves = fwd(bc, cache, l, lgd[t, l][None, :], xs[t], slot_pool, stride)
        ys.append(y.clone())
torch.cuda.synchronize()
h = hashlib.sha256()
for y in ys:
    h.update(y.view(torch.int16).cpu().numpy().tobytes())
keys, ticks = cache.state()
s = hashlib.sha256(np.asarray(keys).tobytes() + np.asarray(ticks).tobytes())
print("outputs", h.hexdigest(), "state", s.hexdigest(), flush=True)
cache.close()
"""


def _run(serialize):
    env = dict(os.environ)
    if serialize:
        env["AMD_SERIALIZE_KERNEL"] = "3"
        env["AMD_SERIALIZE_COPY"] = "3"
    print(f"serialize={serialize}", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("outputs ")]
    assert line, r.stdout[-2000:]
    return line[-1]


def test_cached_trace_serialized_equals_async():
    a = _run(False)
    b = _run(True)
    assert a == b, (a, b)
