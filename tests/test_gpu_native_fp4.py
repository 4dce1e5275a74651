"""GPU parity of the native FP4 path (MOE_MXFP4_A8): MXFP4 weights against MXFP8
activations on the scaled FP4 x FP8 MFMA, for the pages' large prefill chunks
("Data Check" claim table, Fig 4a row: 8,192-token chunks).

* The activation quantizer is integer work decided by exact arithmetic (a power-
  of-two scale and round-to-nearest-even): its E4M3 codes and E8M0 scales must
  equal the oracle's bit for bit.
* The layer against the oracle's MXFP4_A8 layer (same quantized activations, fp64
  arithmetic): the same bounds as the exact path (2e-2 * RMS on the f32 output,
  plus the bf16 half-ulp on the bf16 output); the GPU's products of E2M1 and E4M3
  values are exact and only the f32 sums and the bf16 intermediate round.
* Against the exact oracle (bf16 activations, no quantization) the difference is
  the MXFP8 rounding of the activations: each element off by up to 2^-4 of its
  value (three mantissa bits, round to nearest; a little more for block maxima
  clamped to 448), 2^-4 / sqrt(3) = 3.6% RMS per element.  The gate and up sums
  carry that relative error, SwiGLU combines the two (about 5%), and the down sum
  averages it: the oracle with and without the quantization differs by 4.2% of
  RMS(y) on these cases, with single outputs up to 6 times that (0.26 RMS(y)).
  Bounds: RMS of the difference <= 0.06 RMS(y), largest <= 0.4 RMS(y).
"""
import numpy as np
import pytest
import torch

import synth
from helpers import (BF16_REL, W_ATOL, W_RTOL, assert_close_rel, bf16_to_f64, check_bf16_output, combine_f32, dev,
                     log, run_resident_layer, to_dev)
from routed_expert_ffn_layer_amd import layer as L
from routed_expert_ffn_layer_amd import moe

pytestmark = pytest.mark.gpu

A8 = moe.MOE_MXFP4_A8
QUANT_RMS, QUANT_MAX = 0.06, 0.4


def test_mx8_quantize_bit_exact(ora):
    g = np.random.default_rng(21)
    T, H = 37, 512
    x = g.standard_normal((T, H)) * np.exp(g.uniform(-8, 8, size=(T, 1)))
    x[0, :32] = 0.0                                       # all-zero block
    x[1, :32] = [1.0, 1.0625 / 256, 1.1875 / 256, 1.5 * 2 ** -9 / 256, 2.5 * 2 ** -9 / 256] + [-0.0] * 27  # ties
    x[2, :32] = 0.25
    x[2, 0] = 1.99                                        # scaled beyond 448: clamps
    x[3, :32] = 3e-39                                     # bf16 subnormals
    x[4, 5] = 3e38                                        # near the top of the range
    xb = synth.bf16_bits(x.astype(np.float32))
    codes = torch.empty((T, H), dtype=torch.uint8, device=dev())
    scales = torch.empty((T, H // 32), dtype=torch.uint8, device=dev())
    moe.moe_mx8_quantize(to_dev(xb), codes, scales)
    torch.cuda.synchronize()
    rc, rs = ora.mx8_quantize(xb)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def _layer(T, H, I, E, k, seed, shared=False, logits="normal"):
    I_sh = 128 if shared else 0
    lay = synth.small_layer(synth.MXFP4, T, H, I, E, k, seed=seed, shared=shared, I_shared=I_sh, logits=logits)
    return dict(lay, dtype=A8)


def _check_a8(ora, lay, b):
    H, I, k = lay["H"], lay["I"], lay["k"]
    ref = ora.layer(A8, lay["experts"], lay["x"], lay["logits"], k, H, I, shared=lay.get("shared"),
                    I_shared=lay.get("I_shared", 0))
    np.testing.assert_array_equal(b.topk_ids.cpu().numpy(), ref["ids"])
    np.testing.assert_allclose(b.topk_w.cpu().numpy(), ref["w"], rtol=W_RTOL, atol=W_ATOL)
    inv = b.inv_rows.cpu().numpy()[: b.T * k]
    rows = b.out_rows.cpu().numpy().astype(np.float64)[inv]
    r = assert_close_rel(rows, ref["rows"], BF16_REL, "expert rows vs the MXFP8-activation oracle")
    if ref["shared_out"] is not None:
        assert_close_rel(b.shared_out.cpu().numpy()[: b.T], ref["shared_out"], BF16_REL, "shared rows")
    check_bf16_output(b, ref["shared_out"] is not None, ref["y"], BF16_REL, "y vs the MXFP8-activation oracle")
    exact = ora.layer(synth.MXFP4, lay["experts"], lay["x"], lay["logits"], k, H, I, shared=lay.get("shared"),
                      I_shared=lay.get("I_shared", 0))
    d = combine_f32(b, ref["shared_out"] is not None) - exact["y"]
    rms = np.sqrt(np.mean(exact["y"] ** 2))
    q_rms, q_max = np.sqrt(np.mean(d ** 2)) / rms, np.abs(d).max() / rms
    log(f"  expert rows err/RMS {r:.2e}; y vs exact-activation oracle: RMS err {q_rms:.3f} (bound {QUANT_RMS}), "
        f"max err {q_max:.3f} (bound {QUANT_MAX}) of RMS(y)")
    assert q_rms <= QUANT_RMS and q_max <= QUANT_MAX


NATIVE_CASES = [
    # (T, H, I, E, k, shared, logits): token counts from 1 to 8 tiles of 32 per
    # pass and beyond (two passes), K = 4096 (two scale words per row), ragged
    # expert sizes, a shared expert
    (300, 256, 128, 4, 2, False, "normal"),
    (40, 512, 256, 8, 3, True, "normal"),
    (700, 256, 128, 2, 1, False, "normal"),
    (220, 4096, 256, 8, 2, False, "zipf"),
    (600, 1024, 384, 16, 4, True, "zipf"),
    # weight-scale windows of 2048 columns: four for K = 8192, a short second one
    # for K = 2176 (gate_up) and 2304 (down)
    (300, 8192, 256, 4, 2, False, "normal"),
    (140, 2176, 2304, 4, 2, True, "zipf"),
]


@pytest.mark.parametrize("case", NATIVE_CASES, ids=lambda c: f"T{c[0]}_H{c[1]}_I{c[2]}_E{c[3]}_k{c[4]}_sh{int(c[5])}_{c[6]}")
def test_native_layers(ora, case):
    T, H, I, E, k, shared, logits = case
    assert moe.moe_grouped_ffn_kind(T, k, E, H, I, 128 if shared else 0, A8) == moe.MOE_FFN_GROUPED_GEMM
    log(f"native FP4 layer T={T} H={H} I={I} E={E} k={k} shared={shared} {logits}")
    lay = _layer(T, H, I, E, k, seed=800 + T, shared=shared, logits=logits)
    b, *_ = run_resident_layer(lay)
    _check_a8(ora, lay, b)


def test_native_unsupported_shape_is_refused():
    assert moe.moe_grouped_ffn_kind(64, 2, 8, 160, 96, 0, A8) == -1


def test_native_prefill_chunk_8192_sampled(ora):
    """The MXFP4 prefill layer shape (H=4096, I=2048, 256 experts, top-6) with an
    8,192-token chunk: about 192 tokens per expert (6 tiles of 32 in one pass).
    Routing and permutation in full; every row of three experts and y of 6 tokens
    against the MXFP8-activation oracle."""
    c = synth.CONFIGS["prefill_mxfp4"]
    H, I, E, k, T = c["H"], c["I"], c["E"], c["k"], 8192
    pool = synth.torch_mxfp4_expert_pool(E, H, I, seed=c["seed"], device=dev())
    stride = pool.shape[1]
    x = synth.encode_activations(synth.MXFP4, synth.normal_x(c["seed"], T, H, 5))
    logits = synth.normal_logits(c["seed"], T, E, 5)
    log(f"native FP4 prefill chunk T={T}")
    b = L.LayerBuffers(T, E, k, H, I, A8)
    L.forward(b, to_dev(logits), to_dev(x), pool, stride, L.identity_slots(E))
    torch.cuda.synchronize()
    ids, _, w64 = ora.route_topk(logits, k)
    np.testing.assert_array_equal(b.topk_ids.cpu().numpy(), ids)
    rc, ro, rs, ri = ora.permute(ids, E)
    np.testing.assert_array_equal(b.sorted_rows.cpu().numpy()[: T * k], rs)
    out_rows = b.out_rows.cpu().numpy().astype(np.float64)
    order = np.argsort(rc)
    chosen = [int(order[0]), int(order[E // 2]), int(order[-1])]   # fewest, median, most tokens
    for e in chosen:
        toks = [int(r) // k for r in rs[ro[e]:ro[e + 1]]]
        log(f"  expert {e}: {len(toks)} tokens")
        ref = ora.expert_rows(A8, pool[e].cpu().numpy(), H, I, x, toks)
        assert_close_rel(out_rows[ro[e]:ro[e + 1]], ref, BF16_REL, f"expert {e} rows ({len(toks)} tokens)")
    sample = sorted(set([0, T - 1] + list(np.random.default_rng(3).choice(T, size=4, replace=False))))
    by_expert = {}
    for t in sample:
        for j in range(k):
            by_expert.setdefault(int(ids[t, j]), []).append(t)
    o_ref = {}
    for e, toks in by_expert.items():
        for t, row in zip(toks, ora.expert_rows(A8, pool[e].cpu().numpy(), H, I, x, toks)):
            o_ref[(t, e)] = row
    y_ref = np.array([sum(w64[t, j] * o_ref[(t, int(ids[t, j]))] for j in range(k)) for t in sample])
    y = combine_f32(b, False)
    r = assert_close_rel(y[sample], y_ref, BF16_REL, "sampled y (f32 output)")
    log(f"  sampled y err/RMS {r:.2e}")
