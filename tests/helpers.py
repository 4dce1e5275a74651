"""Helpers of the GPU parity tests: upload seeded inputs, run the library through
the C ABI, compare with the oracle."""
import sys

import numpy as np
import torch

import synth
from routed_expert_ffn_layer_amd import layer as L
from routed_expert_ffn_layer_amd import moe

# Float tolerances: f32 layers max-abs <= 1e-4; bf16 / MXFP4 layers
# max-abs <= 2e-2 * RMS(oracle output).  Gate weights (f32 softmax vs fp64):
W_RTOL, W_ATOL = 2e-6, 1e-7
F32_ATOL = 1e-4
BF16_REL = 2e-2


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def pool_from_experts(experts, stride=None):
    """uint8 [E][expert_bytes] -> device pool with 256-byte aligned slot stride."""
    E, nb = experts.shape
    stride = stride or ((nb + 255) // 256) * 256
    pool = torch.zeros((E, stride), dtype=torch.uint8, device=dev())
    pool[:, :nb] = to_dev(experts)
    return pool, stride


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close_rel(got, ref, rel=BF16_REL, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= rel * rms, f"{what}: max abs err {err:.3e} > {rel} * RMS {rms:.3e}"
    return err / rms if rms else 0.0


def assert_close_abs(got, ref, atol=F32_ATOL, what=""):
    err = float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64)))) if np.size(ref) else 0.0
    assert err <= atol, f"{what}: max abs err {err:.3e} > {atol}"
    return err


def bf16_rne(a):
    """float64/float32 -> nearest-even bf16 values (as float64)."""
    return synth.bf16_bits_to_f32(synth.bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


def combine_f32(b, with_shared):
    """Re-run the combine of buffers b with an f32 output (the bf16 output of the
    same call is its round-to-nearest-even, checked separately)."""
    y32 = torch.empty((b.T, b.H), dtype=torch.float32, device=dev())
    moe.moe_combine(b.out_rows, b.topk_w, b.inv_rows, b.shared_out if with_shared else None, y32, moe.MOE_F32)
    torch.cuda.synchronize()
    return y32.cpu().numpy()


def bf16_half_ulp(v):
    """Half a bf16 unit in the last place at |v| (7 stored mantissa bits): the
    largest error of rounding an exact value v to bf16."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def assert_close_bf16_output(got, ref, rel=BF16_REL, what=""):
    """A bf16 output against the exact value: |got - ref| <= rel * RMS(ref) plus the
    half-ulp of bf16 at ref, element by element (an exact result rounded to bf16
    is off by up to that half-ulp, which at |y| ~ 5 RMS is itself ~2% of RMS).
    Returns the largest error beyond the half-ulp, over RMS."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    excess = np.abs(got - ref) - bf16_half_ulp(ref)
    worst = float(excess.max()) if ref.size else 0.0
    assert worst <= rel * rms, f"{what}: error beyond the bf16 half-ulp {worst:.3e} > {rel} * RMS {rms:.3e}"
    return worst / rms if rms else 0.0


def check_bf16_output(b, with_shared, ref_y, rel=BF16_REL, what="y"):
    """bf16 layer output.  The same call with an f32 output (the library's other
    output type) within rel * RMS of the oracle; the bf16 output bitwise the
    round-to-nearest-even of it, and within rel * RMS plus its own rounding
    (half a bf16 ulp) of the oracle.  The ratios are logged, so the margin left
    under the bound is visible."""
    y32 = combine_f32(b, with_shared)
    y16 = bf16_to_f64(b.y)
    np.testing.assert_array_equal(y16, bf16_rne(y32))
    r32 = assert_close_rel(y32, ref_y, rel, what + " (f32 output)")
    r16 = assert_close_bf16_output(y16, ref_y, rel, what + " (bf16 output)")
    rms = float(np.sqrt(np.mean(np.asarray(ref_y, np.float64) ** 2)))
    raw = float(np.max(np.abs(y16 - ref_y))) / rms if rms else 0.0
    log(f"{what}: max err / RMS = {r32:.2e} (f32 output), {raw:.2e} (bf16 output, {r16:.2e} beyond its "
        f"half-ulp); bound {rel:.0e}")
    return r32


def run_resident_layer(lay, stream=None):
    """lay: dict from synth.small_layer / tiny_layer.  Returns (buffers, torch y)."""
    T, E = lay["logits"].shape
    dtype = lay.get("dtype", synth.F32)
    cfg = lay.get("cfg", {})
    H = lay.get("H", cfg.get("H"))
    I = lay.get("I", cfg.get("I"))
    k = lay.get("k", cfg.get("k"))
    I_sh = lay.get("I_shared", 0)
    b = L.LayerBuffers(T, E, k, H, I, dtype, I_shared=I_sh)
    pool, stride = pool_from_experts(lay["experts"])
    sh = to_dev(lay["shared"]) if lay.get("shared") is not None else None
    x = to_dev(lay["x"])
    logits = to_dev(lay["logits"])
    L.forward(b, logits, x, pool, stride, L.identity_slots(E), sh, stream)
    torch.cuda.synchronize()
    return b, pool, stride, sh, x, logits
