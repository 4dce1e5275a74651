"""The five layer workloads: shapes and seeded input recipes.

Base seed of workload n (n = 0..4 in the order below) is 1000 + n + 1; every draw
uses its own numpy SeedSequence substream keyed by (purpose, layer, batch, ...).

The pages describe DeepSeek-V4-Flash as 6 of 256 routed experts in each of 43
layers and a 37% cache capacity (page "Meet FreeToken: An Edge-Native MoE Serving
Engine ..." (MarkTechPost), sections "The gap it targets" and "Results"); the
remaining shape numbers are the workload definitions below.
"""
import math
import numpy as np

from .gen import F32, BF16, MXFP4, rng, random_expert, encode_activations, expert_bytes

# purpose keys for substreams
_X, _LOGITS, _WEIGHTS, _ROUTER, _PERM, _TRACE, _SHARED = 1, 2, 3, 4, 5, 6, 7

CONFIGS = {
    "tiny_f32": dict(name="tiny_f32", seed=1001, dtype=F32, T=32, H=256, I=512, E=8, k=2,
                     shared=False, I_shared=0, n_slots=4, layers=1),
    "decode_bf16": dict(name="decode_bf16", seed=1002, dtype=BF16, T_list=(1, 4, 16), H=2048, I=512,
                        E=256, k=8, shared=True, I_shared=512, layers=1),
    "decode_mxfp4": dict(name="decode_mxfp4", seed=1003, dtype=MXFP4, T_list=(1, 8, 64), H=4096, I=2048,
                         E=256, k=6, shared=False, I_shared=0, layers=43, zipf_s=1.1),
    "prefill_mxfp4": dict(name="prefill_mxfp4", seed=1004, dtype=MXFP4, T=4096, H=4096, I=2048,
                          E=256, k=6, shared=False, I_shared=0, layers=43),
    "cached_trace_bf16": dict(name="cached_trace_bf16", seed=1005, dtype=BF16, tokens=1000, H=2048, I=512,
                              E=256, k=8, shared=False, I_shared=0, layers=48, reuse_p=0.7, zipf_s=1.0,
                              capacity_frac=0.37),
}


def cache_slots_for(cfg) -> int:
    """Slots of the cached-trace workload: floor(capacity_frac * layers * E)."""
    return int(math.floor(cfg["capacity_frac"] * cfg["layers"] * cfg["E"]))


def normal_logits(seed, T, E, *path):
    """Router logits ~ N(0,1) iid, f32 [T][E]."""
    return rng(seed, _LOGITS, *path).standard_normal((T, E)).astype(np.float32)


def normal_x(seed, T, H, *path):
    """Token activations ~ N(0,1), f32 [T][H] (encode with encode_activations)."""
    return rng(seed, _X, *path).standard_normal((T, H)).astype(np.float32)


def popularity_perm(seed, layer, E):
    """Seeded per-layer permutation pi_l: expert e has popularity rank pi_l(e) (0 = hottest)."""
    return rng(seed, _PERM, layer).permutation(E)


def zipf_noise_logits(seed, T, E, layer, s, batch=0):
    """logits[t,e] = -s*ln(1 + pi_l(e)) + N(0,1): Zipf(s)-skewed popularity plus noise."""
    pi = popularity_perm(seed, layer, E)
    base = -s * np.log1p(pi.astype(np.float64))
    noise = rng(seed, _LOGITS, layer, batch).standard_normal((T, E))
    return (base[None, :] + noise).astype(np.float32)


def trace_logits(seed, tokens, layers, E, s=1.0, reuse_p=0.7):
    """Temporally correlated routing trace, f32 [tokens][layers][E].

    Per (t, l): with probability reuse_p (t > 0) the row of token t-1 is reused, so
    the token takes the previous token's expert set; otherwise
    logits = -s*ln(1 + pi_l(e)) + Gumbel(0,1), whose top-k is an exact draw without
    replacement from the Zipf(s) popularity (the Gumbel-top-k construction).
    """
    out = np.empty((tokens, layers, E), dtype=np.float32)
    for l in range(layers):
        pi = popularity_perm(seed, l, E)
        base = -s * np.log1p(pi.astype(np.float64))
        g = rng(seed, _TRACE, l)
        reuse = g.random(tokens) < reuse_p
        gum = g.gumbel(size=(tokens, E))
        for t in range(tokens):
            if t > 0 and reuse[t]:
                out[t, l] = out[t - 1, l]
            else:
                out[t, l] = (base + gum[t]).astype(np.float32)
    return out


def tiny_layer(cfg=None):
    """The tiny f32 layer: x, router-projected logits, and E experts' slot bytes.

    logits = x . W_r^T is evaluated here once in float64 and rounded to f32; both
    sides of every comparison consume the same f32 logits.
    """
    cfg = cfg or CONFIGS["tiny_f32"]
    s, T, H, I, E = cfg["seed"], cfg["T"], cfg["H"], cfg["I"], cfg["E"]
    x = normal_x(s, T, H)
    w_r = rng(s, _ROUTER).standard_normal((E, H)) * 0.02
    logits = (x.astype(np.float64) @ w_r.T).astype(np.float32)
    experts = np.stack([random_expert(F32, H, I, rng(s, _WEIGHTS, 0, e)) for e in range(E)])
    return dict(x=encode_activations(F32, x), x_f32=x, logits=logits, experts=experts, cfg=cfg)


def small_layer(dtype, T, H, I, E, k, seed, shared=False, I_shared=0, logits="normal", layer=0, zipf_s=1.1):
    """A generic seeded layer (for parity tests at sizes the oracle finishes quickly)."""
    x = normal_x(seed, T, H, layer)
    if logits == "normal":
        lg = normal_logits(seed, T, E, layer)
    else:
        lg = zipf_noise_logits(seed, T, E, layer, zipf_s)
    experts = np.stack([random_expert(dtype, H, I, rng(seed, _WEIGHTS, layer, e)) for e in range(E)])
    sh = random_expert(dtype, H, I_shared, rng(seed, _SHARED, layer)) if shared else None
    return dict(x=encode_activations(dtype, x), x_f32=x, logits=lg, experts=experts, shared=sh,
                dtype=dtype, T=T, H=H, I=I, E=E, k=k, I_shared=I_shared if shared else 0)


__all__ = ["CONFIGS", "cache_slots_for", "normal_logits", "normal_x", "popularity_perm",
           "zipf_noise_logits", "trace_logits", "tiny_layer", "small_layer", "expert_bytes",
           "F32", "BF16", "MXFP4"]
