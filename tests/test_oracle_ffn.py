"""Pins of the oracle's SwiGLU expert FFN, combine and whole layer.

Independent checks: textbook SiLU values, numpy matmul with scipy's logistic
function, exact scaling invariants, special cases that collapse the layer to a
dense FFN or to a single expert, and a pure-Python loop on a tiny shape.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import synth

SIG1 = 0.7310585786300049  # logistic(1), textbook value


def _dense_ffn(wg, wu, wd, x):
    a = wg @ x
    b = wu @ x
    return wd @ (a * expit(a) * b)


def test_silu_applies_to_gate_not_up(ora):
    # x = e0; gate column 0 = g, up column 0 = u; down = identity on the first I rows
    H, I = 4, 3
    wg = np.zeros((I, H)); wu = np.zeros((I, H)); wd = np.zeros((H, I))
    wg[:, 0] = [1.0, -1.0, 0.0]
    wu[:, 0] = [2.0, 2.0, 5.0]
    for j in range(I):
        wd[j, j] = 1.0
    o = ora.expert_ffn(wg, wu, wd, np.array([1.0, 0, 0, 0]))
    assert o[0] == pytest.approx(SIG1 * 2.0, rel=1e-15)          # silu(1) * 2
    assert o[1] == pytest.approx(-(1 - SIG1) * 2.0, rel=1e-15)   # silu(-1) * 2
    assert o[2] == 0.0                                          # silu(0) * 5
    assert o[3] == 0.0


def test_down_projection_orientation(ora):
    # H != I; a single nonzero in Wd at (row 2, col 1) routes h[1] to o[2] only
    H, I = 5, 3
    wg = np.zeros((I, H)); wu = np.zeros((I, H)); wd = np.zeros((H, I))
    wg[1, 4] = 1.0
    wu[1, 4] = 1.0
    wd[2, 1] = 3.0
    x = np.zeros(H); x[4] = 1.0
    o = ora.expert_ffn(wg, wu, wd, x)
    exp = np.zeros(H); exp[2] = 3.0 * SIG1
    np.testing.assert_allclose(o, exp, rtol=1e-15, atol=0)


def test_ffn_matches_numpy_and_pure_python(ora):
    g = np.random.default_rng(1)
    H, I = 48, 40
    wg = g.standard_normal((I, H)) * 0.2
    wu = g.standard_normal((I, H)) * 0.2
    wd = g.standard_normal((H, I)) * 0.2
    x = g.standard_normal(H)
    o = ora.expert_ffn(wg, wu, wd, x)
    np.testing.assert_allclose(o, _dense_ffn(wg, wu, wd, x), rtol=1e-12, atol=1e-14)
    # pure Python on a slice of the problem
    h = []
    for j in range(I):
        a = sum(wg[j][c] * x[c] for c in range(H))
        b = sum(wu[j][c] * x[c] for c in range(H))
        h.append(a / (1 + math.exp(-a)) * b)
    for r in range(0, H, 7):
        assert o[r] == pytest.approx(sum(wd[r][j] * h[j] for j in range(I)), rel=1e-12, abs=1e-14)


def _layer(ora, dtype, T, H, I, E, k, seed, shared=False, same_expert=False, zero=False):
    L = synth.small_layer(dtype, T, H, I, E, k, seed, shared=shared, I_shared=I if shared else 0)
    experts = L["experts"]
    if same_expert:
        experts = np.stack([experts[0]] * E)
    if zero:
        experts = np.zeros_like(experts)
    out = ora.layer(dtype, experts, L["x"], L["logits"], k, H, I, shared=L["shared"], I_shared=L["I_shared"])
    return L, experts, out


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_identical_experts_reduce_to_dense_ffn(ora, dtype):
    T, H, I, E, k = 6, 64, 32, 8, 3
    L, experts, out = _layer(ora, dtype, T, H, I, E, k, seed=21, same_expert=True)
    wg, wu, wd = ora.decode_expert(dtype, experts[0], H, I)
    x = ora.decode_x(dtype, L["x"], T, H)
    for t in range(T):
        np.testing.assert_allclose(out["y"][t], _dense_ffn(wg, wu, wd, x[t]), rtol=1e-11, atol=1e-13)


def test_zero_weights_give_zero(ora):
    _, _, out = _layer(ora, 1, 4, 64, 32, 8, 2, seed=3, zero=True)
    assert np.all(out["y"] == 0.0)


def test_doubling_down_projection_doubles_output_exactly(ora):
    T, H, I, E, k = 5, 64, 32, 6, 2
    L, experts, out = _layer(ora, 0, T, H, I, E, k, seed=9)
    doubled = experts.copy()
    w = doubled[:, 2 * I * H * 4:].view(np.float32)
    w *= 2.0
    out2 = ora.layer(0, doubled, L["x"], L["logits"], k, H, I)
    np.testing.assert_array_equal(out2["y"], 2.0 * out["y"])


def test_mxfp4_scale_increment_doubles_output_exactly(ora):
    T, H, I, E, k = 4, 64, 32, 4, 2
    L, experts, out = _layer(ora, 2, T, H, I, E, k, seed=10)
    bumped = experts.copy()
    bumped[:, synth.slot_offsets(synth.MXFP4, H, I)["s2"]:] += 1
    out2 = ora.layer(2, bumped, L["x"], L["logits"], k, H, I)
    np.testing.assert_array_equal(out2["y"], 2.0 * out["y"])


def test_k1_gives_the_chosen_expert_row(ora):
    T, H, I, E = 5, 32, 32, 4
    L, experts, out = _layer(ora, 1, T, H, I, E, 1, seed=12)
    x = ora.decode_x(1, L["x"], T, H)
    for t in range(T):
        e = out["ids"][t, 0]
        wg, wu, wd = ora.decode_expert(1, experts[e], H, I)
        np.testing.assert_allclose(out["y"][t], _dense_ffn(wg, wu, wd, x[t]), rtol=1e-11, atol=1e-13)


def test_layer_equals_weighted_sum_with_shared(ora):
    T, H, I, E, k = 4, 32, 32, 6, 3
    L, experts, out = _layer(ora, 1, T, H, I, E, k, seed=14, shared=True)
    x = ora.decode_x(1, L["x"], T, H)
    sg, su, sd = ora.decode_expert(1, L["shared"], H, I)
    ids, _, w64 = ora.route_topk(L["logits"], k)
    for t in range(T):
        ref = _dense_ffn(sg, su, sd, x[t])
        for j in range(k):
            wg, wu, wd = ora.decode_expert(1, experts[ids[t, j]], H, I)
            ref = ref + w64[t, j] * _dense_ffn(wg, wu, wd, x[t])
        np.testing.assert_allclose(out["y"][t], ref, rtol=1e-11, atol=1e-13)


def test_combine_closed_form(ora):
    rows = np.arange(2 * 3 * 4, dtype=np.float64).reshape(6, 4)
    w = np.array([[0.5, 0.25, 0.25], [1.0, 0.0, 0.0]])
    shared = np.ones((2, 4))
    y = ora.combine(rows, w, shared)
    np.testing.assert_array_equal(y[0], 0.5 * rows[0] + 0.25 * rows[1] + 0.25 * rows[2] + 1)
    np.testing.assert_array_equal(y[1], rows[3] + 1)
