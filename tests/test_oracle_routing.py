"""Pins of the oracle's top-k gating and permutation.

Top-k is checked against numpy's stable argsort and a pure-Python sort; the gate
weights against closed forms and against softmax-over-all-E-then-renormalise
(scipy); the permutation against a brute-force sort by (expert, pair index).
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import synth


def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(8, 1), (8, 2), (64, 6), (256, 8), (256, 6), (100, 7)])
def test_topk_matches_stable_argsort(ora, E, k):
    g = np.random.default_rng(E * 31 + k)
    logits = g.standard_normal((40, E)).astype(np.float32)
    ids, w32, w64 = ora.route_topk(logits, k)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(ids, ref)
    for t in range(5):
        assert list(ids[t]) == _brute_topk(logits[t], k)


def test_topk_forced_ties_go_to_lower_index(ora):
    g = np.random.default_rng(7)
    logits = g.integers(0, 3, size=(200, 16)).astype(np.float32)
    for k in (1, 3, 8, 16):
        ids, _, _ = ora.route_topk(logits, k)
        ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        np.testing.assert_array_equal(ids, ref)
        for t in range(20):
            assert list(ids[t]) == _brute_topk(logits[t], k)


def test_topk_all_equal_rows(ora):
    for k in (1, 2, 8):
        ids, w32, w64 = ora.route_topk(np.full((3, 32), 1.25, np.float32), k)
        np.testing.assert_array_equal(ids, np.tile(np.arange(k), (3, 1)))
        # equal logits -> exactly 1/k (k a power of two)
        assert np.all(w64 == 1.0 / k) and np.all(w32 == np.float32(1.0 / k))


def test_topk_signed_zero_is_a_tie(ora):
    row = np.array([[-0.0, 0.0, -1.0, -0.0]], np.float32)
    ids, _, _ = ora.route_topk(row, 3)
    assert list(ids[0]) == [0, 1, 3]


def test_topk_k_equals_E_gives_full_order(ora):
    g = np.random.default_rng(11)
    logits = g.standard_normal((10, 12)).astype(np.float32)
    ids, _, _ = ora.route_topk(logits, 12)
    np.testing.assert_array_equal(ids, np.argsort(-logits, axis=1, kind="stable"))


def test_topk_rejects_nan_and_inf(ora):
    for bad in (np.nan, np.inf, -np.inf):
        l = np.zeros((2, 8), np.float32)
        l[1, 3] = bad
        with pytest.raises(ora.OracleError):
            ora.route_topk(l, 2)


def test_gate_weights_closed_forms(ora):
    g = np.random.default_rng(5)
    logits = g.standard_normal((50, 64)).astype(np.float32) * 3
    ids, w32, w64 = ora.route_topk(logits, 1)
    assert np.all(w64 == 1.0) and np.all(w32 == 1.0)
    for k in (2, 6, 8):
        ids, w32, w64 = ora.route_topk(logits, k)
        assert np.all(np.abs(w64.sum(1) - 1.0) <= k * 2.0 ** -52)
        # equal to softmax over all E followed by renormalising the selected k
        p = softmax(logits.astype(np.float64), axis=1)
        sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
        ref = sel / sel.sum(1, keepdims=True)
        np.testing.assert_allclose(w64, ref, rtol=1e-13, atol=0)
        # weights are non-increasing along the choice order
        assert np.all(np.diff(w64, axis=1) <= 0)
        # f32 weights are the fp64 weights rounded to nearest
        np.testing.assert_array_equal(w32, w64.astype(np.float32))


def test_gate_weights_two_way_closed_form(ora):
    # two selected logits a > b: w0 = 1 / (1 + e^(b - a))
    logits = np.array([[0.0, 2.0, -5.0, 1.0]], np.float32)
    ids, _, w64 = ora.route_topk(logits, 2)
    assert list(ids[0]) == [1, 3]
    assert w64[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert w64[0, 1] == pytest.approx(1.0 / (1.0 + math.exp(1.0)), rel=1e-15)


@pytest.mark.parametrize("T,k,E", [(1, 8, 256), (16, 8, 256), (32, 2, 8), (300, 6, 256), (5, 3, 1000)])
def test_permute_matches_brute_force(ora, T, k, E):
    g = np.random.default_rng(T * 7 + E)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_rows, inv_rows = ora.permute(ids, E)
    flat = ids.ravel()
    brute = sorted(range(T * k), key=lambda r: (int(flat[r]), r))
    np.testing.assert_array_equal(sorted_rows, brute)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    assert counts.sum() == T * k and offsets[E] == T * k and offsets[0] == 0
    np.testing.assert_array_equal(np.diff(offsets), counts)
    np.testing.assert_array_equal(inv_rows[sorted_rows], np.arange(T * k))
    np.testing.assert_array_equal(sorted_rows[inv_rows], np.arange(T * k))
    for e in range(E):
        seg = sorted_rows[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_permute_empty(ora):
    counts, offsets, s, inv = ora.permute(np.zeros((0, 4), np.int32), 16)
    assert counts.sum() == 0 and np.all(offsets == 0) and s.size == 0 and inv.size == 0


def test_router_logits_against_float64_matmul(ora):
    """The router projection equals a float64 matrix product of the decoded bf16
    inputs (numpy), to fp64 rounding."""
    g = np.random.default_rng(21)
    T, H, E = 5, 96, 24
    x = synth.bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    wr = synth.bf16_bits((g.standard_normal((E, H)) * 0.02).astype(np.float32))
    got = ora.router_logits(x, wr)
    ref = synth.bf16_bits_to_f32(x).astype(np.float64) @ synth.bf16_bits_to_f32(wr).astype(np.float64).T
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)


def test_router_logits_closed_forms(ora):
    g = np.random.default_rng(22)
    H, E = 64, 10
    wr = synth.bf16_bits((g.standard_normal((E, H)) * 0.02).astype(np.float32))
    w = synth.bf16_bits_to_f32(wr).astype(np.float64)
    # a one-hot token picks one column of the router exactly
    x = np.zeros((1, H), np.float32); x[0, 17] = 1.0
    np.testing.assert_array_equal(ora.router_logits(synth.bf16_bits(x), wr)[0], w[:, 17])
    # scaling a token by 2 doubles every logit exactly; the zero token gives zeros
    xs = synth.bf16_bits(g.standard_normal((3, H)).astype(np.float32))
    l1 = ora.router_logits(xs, wr)
    x2 = synth.bf16_bits(2 * synth.bf16_bits_to_f32(xs))
    np.testing.assert_array_equal(ora.router_logits(x2, wr), 2 * l1)
    np.testing.assert_array_equal(ora.router_logits(np.zeros((2, H), np.uint16), wr), np.zeros((2, E)))
