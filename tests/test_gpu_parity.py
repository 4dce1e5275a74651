"""GPU parity: every kernel through the C ABI against the fp64 CPU oracle.

Integer outputs (expert ids, permutation, cache state) must be bit-exact; gate
weights within f32 rounding; layer outputs within max-abs 1e-4 (f32 layers) or
2e-2 * RMS(oracle output) (bf16 and MXFP4 layers).
"""
import numpy as np
import pytest
import torch

import synth
from helpers import (BF16_REL, F32_ATOL, W_ATOL, W_RTOL, assert_close_abs, assert_close_bf16_output, assert_close_rel,
                     bf16_rne, bf16_to_f64,
                     check_bf16_output, combine_f32, dev, log, pool_from_experts, run_resident_layer, to_dev)
from routed_expert_ffn_layer_amd import layer as L
from routed_expert_ffn_layer_amd import moe

pytestmark = pytest.mark.gpu


def _topk_gpu(logits, k):
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=dev())
    w = torch.empty((T, k), dtype=torch.float32, device=dev())
    moe.moe_route_topk(to_dev(logits), k, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _topk_cases():
    g = np.random.default_rng(100)
    yield "tiny", synth.tiny_layer()["logits"], 2
    for T in (1, 4, 16):
        yield f"decode_T{T}", synth.normal_logits(1002, T, 256, 0), 8
    yield "zipf_T64", synth.zipf_noise_logits(1003, 64, 256, 5, 1.1), 6
    yield "prefill_T4096", synth.normal_logits(1004, 4096, 256, 0), 6
    yield "ties_int", g.integers(0, 3, size=(300, 256)).astype(np.float32), 8
    yield "all_equal", np.full((7, 100), 0.5, np.float32), 5
    yield "signed_zero", np.array([[-0.0, 0.0, -1.0, -0.0] + [-2.0] * 60], np.float32), 3
    yield "E8_k8", g.standard_normal((33, 8)).astype(np.float32), 8
    yield "E100_k1", g.standard_normal((65, 100)).astype(np.float32), 1
    yield "E1024_k32", g.standard_normal((9, 1024)).astype(np.float32), 32
    yield "E513_k16_ties", g.integers(-2, 2, size=(20, 513)).astype(np.float32), 16


@pytest.mark.parametrize("case", list(_topk_cases()), ids=lambda c: c[0])
def test_topk_matches_oracle(ora, case):
    name, logits, k = case
    log(f"topk case {name} T={logits.shape[0]} E={logits.shape[1]} k={k}")
    ids, w = _topk_gpu(logits, k)
    rids, _, rw = ora.route_topk(logits, k)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=W_RTOL, atol=W_ATOL)


@pytest.mark.parametrize("T,k,E", [(0, 4, 16), (1, 8, 256), (8, 6, 256), (64, 16, 1024), (65, 6, 256), (17, 2, 8),
                                   (300, 8, 256), (5, 1, 1), (40, 3, 100),
                                   # small-batch kernel (T <= 8, T*k <= 64): exactly 64 pairs, E = 1024,
                                   # ragged E, k = 32; the larger fused kernel: 8 tokens of 16 pairs
                                   (8, 8, 256), (2, 16, 1024), (3, 4, 300), (1, 32, 64), (7, 9, 40), (64, 1, 64),
                                   (8, 16, 256)])
def test_route_fused_matches_separate_calls_and_oracle(ora, T, k, E):
    """moe_route (one launch up to 8 tokens: a register permutation up to 64
    (token, expert) pairs, else the workgroup one; separate launches above) =
    moe_route_topk + moe_permute bit for bit,
    and the oracle's routing and permutation; logits rounded to a coarse grid so
    that ties occur."""
    log(f"route T={T} k={k} E={E}")
    g = np.random.default_rng(900 + T + E)
    logits = (np.round(g.standard_normal((T, E)) * 4) / 4).astype(np.float32)
    lg = to_dev(logits) if T else torch.zeros((0, E), dtype=torch.float32, device=dev())
    n = max(T * k, 1)

    def bufs():
        return (torch.full((max(T, 1), k), -7, dtype=torch.int32, device=dev()),
                torch.zeros((max(T, 1), k), dtype=torch.float32, device=dev()),
                torch.full((E,), -7, dtype=torch.int32, device=dev()),
                torch.full((E + 1,), -7, dtype=torch.int32, device=dev()),
                torch.full((n,), -7, dtype=torch.int32, device=dev()),
                torch.full((n,), -7, dtype=torch.int32, device=dev()))

    a, b = bufs(), bufs()
    moe.moe_route(lg, k, *a)
    if T:
        moe.moe_route_topk(lg, k, b[0], b[1])
    moe.moe_permute(b[0][:T], E, b[2], b[3], b[4], b[5])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    if T:
        rids, _, rw = ora.route_topk(logits, k)
        np.testing.assert_array_equal(a[0].cpu().numpy(), rids)
        np.testing.assert_allclose(a[1].cpu().numpy(), rw, rtol=W_RTOL, atol=W_ATOL)
        rc, ro, rs, ri = ora.permute(rids, E)
        np.testing.assert_array_equal(a[2].cpu().numpy(), rc)
        np.testing.assert_array_equal(a[3].cpu().numpy(), ro)
        np.testing.assert_array_equal(a[4].cpu().numpy()[:T * k], rs)
        np.testing.assert_array_equal(a[5].cpu().numpy()[:T * k], ri)


@pytest.mark.parametrize("T,k,E", [(0, 4, 16), (1, 8, 256), (16, 8, 256), (32, 2, 8), (4096, 6, 256), (3, 1, 1),
                                   (1000, 32, 1024), (777, 5, 300)])
def test_permute_matches_oracle(ora, T, k, E):
    log(f"permute T={T} k={k} E={E}")
    g = np.random.default_rng(T + E)
    ids = (np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
           if T else np.zeros((0, k), np.int32))
    counts = torch.empty(E, dtype=torch.int32, device=dev())
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev())
    n = max(T * k, 1)
    srt = torch.full((n,), -7, dtype=torch.int32, device=dev())
    inv = torch.full((n,), -7, dtype=torch.int32, device=dev())
    moe.moe_permute(to_dev(ids), E, counts, offsets, srt, inv)
    torch.cuda.synchronize()
    rc, ro, rs, ri = ora.permute(ids, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro)
    np.testing.assert_array_equal(srt.cpu().numpy()[:T * k], rs)
    np.testing.assert_array_equal(inv.cpu().numpy()[:T * k], ri)


def _check_layer(ora, lay, b, rel=None):
    """Compare ids, weights, permutation, expert rows, shared rows and y with the oracle."""
    dtype = lay["dtype"]
    H, I, k = lay["H"], lay["I"], lay["k"]
    ref = ora.layer(dtype, lay["experts"], lay["x"], lay["logits"], k, H, I, shared=lay.get("shared"),
                    I_shared=lay.get("I_shared", 0))
    np.testing.assert_array_equal(b.topk_ids.cpu().numpy(), ref["ids"])
    np.testing.assert_allclose(b.topk_w.cpu().numpy(), ref["w"], rtol=W_RTOL, atol=W_ATOL)
    inv = b.inv_rows.cpu().numpy()[: b.T * k]
    rows = b.out_rows.cpu().numpy().astype(np.float64)[inv]
    if dtype == synth.F32:
        assert_close_abs(rows, ref["rows"], F32_ATOL, "expert rows")
        assert_close_abs(b.y.cpu().numpy(), ref["y"], F32_ATOL, "y")
    else:
        assert_close_rel(rows, ref["rows"], rel or BF16_REL, "expert rows")
        if ref["shared_out"] is not None:
            assert_close_rel(b.shared_out.cpu().numpy()[: b.T], ref["shared_out"], rel or BF16_REL, "shared rows")
        check_bf16_output(b, ref["shared_out"] is not None, ref["y"], rel or BF16_REL)
    return ref


def test_tiny_f32_layer(ora):
    lay = synth.tiny_layer()
    cfg = lay["cfg"]
    lay = dict(lay, dtype=synth.F32, H=cfg["H"], I=cfg["I"], k=cfg["k"], shared=None, I_shared=0)
    log("tiny f32 layer T=32 H=256 I=512 E=8 k=2")
    b, *_ = run_resident_layer(lay)
    _check_layer(ora, lay, b)


# (dtype, T, H, I, E, k, shared, logits, kernel family): ragged token counts,
# several token tiles, more than 128 tokens on one expert (two passes), K not a
# multiple of the MXFP4 step, row-tile counts that leave a block partly filled.
# The kernel family (S: weight streaming, G: grouped GEMM) is asserted against the
# library's dispatch for each case, so a case cannot silently change family.
SMALL = [
    (synth.BF16, 1, 256, 128, 16, 4, True, "normal", "S"),
    (synth.BF16, 5, 256, 128, 16, 4, True, "normal", "S"),
    (synth.BF16, 40, 512, 256, 32, 6, True, "normal", "S"),
    (synth.BF16, 300, 256, 128, 2, 1, False, "normal", "G"),
    (synth.BF16, 70, 128, 64, 4, 4, False, "normal", "S"),
    (synth.MXFP4, 8, 512, 256, 8, 3, False, "normal", "S"),
    (synth.MXFP4, 3, 160, 96, 8, 2, True, "normal", "S"),
    (synth.MXFP4, 33, 256, 128, 16, 6, True, "normal", "S"),
    (synth.MXFP4, 200, 128, 64, 2, 1, False, "normal", "S"),
    (synth.MXFP4, 40, 160, 96, 8, 3, True, "normal", "S"),     # 4-tile down blocks over 10 row tiles: ragged last block
    (synth.BF16, 20, 160, 96, 8, 3, True, "normal", "S"),
    (synth.F32, 9, 64, 32, 5, 2, True, "normal", "S"),
    # grouped GEMM (>= 32 pairs per expert on average, dimensions multiples of 128)
    (synth.BF16, 512, 256, 256, 8, 2, False, "normal", "G"),
    (synth.BF16, 300, 384, 128, 4, 2, True, "normal", "S"),
    (synth.MXFP4, 600, 512, 256, 16, 4, True, "normal", "G"),
    (synth.MXFP4, 257, 256, 384, 8, 1, False, "normal", "G"),
    # grouped GEMM at H = 4096 (two MXFP4 scale blocks per gate_up row tile) with
    # per-expert token counts 63..86, 90..109 and (Zipf-skewed) 5..166
    (synth.MXFP4, 300, 4096, 256, 8, 2, False, "normal", "G"),
    (synth.MXFP4, 400, 4096, 256, 8, 2, False, "normal", "G"),
    (synth.MXFP4, 220, 4096, 256, 8, 2, True, "zipf", "G"),
    (synth.BF16, 300, 4096, 256, 8, 2, False, "zipf", "G"),
    # MXFP4 weight scales staged in LDS 32 chunks (2048 columns) at a time, two
    # windows alternating: gate_up K = 8192 (four windows, each set refilled), and
    # K = 2176 / 2304 (a second window of 2 and 4 chunks), shared down K = 1152
    (synth.MXFP4, 300, 8192, 256, 8, 2, False, "normal", "G"),
    (synth.MXFP4, 140, 2176, 2304, 4, 2, True, "zipf", "G"),
    # MXFP4 weight streaming with whole 16-step scale blocks (K = 2048): one and two
    # token tiles, a shared expert whose down K (1024) is half a block, and a
    # Zipf-skewed batch whose hottest expert carries 98 tokens (several passes)
    (synth.MXFP4, 24, 2048, 2048, 4, 2, False, "normal", "S"),
    (synth.MXFP4, 6, 2048, 2048, 3, 2, True, "normal", "S"),
    (synth.MXFP4, 120, 2048, 512, 8, 2, False, "zipf", "S"),
    # token rows staged in LDS with K not a multiple of 128 (clamped columns), shared expert
    (synth.MXFP4, 5, 160, 96, 8, 2, True, "normal", "S"),
    # H = 4096: the launch's LDS holds 5 token rows, so experts with more tokens (and
    # the shared expert) read theirs from memory in the same launch
    (synth.MXFP4, 12, 4096, 256, 4, 2, True, "normal", "S"),
]


def _small_id(c):
    return f"{synth.DTYPE_NAMES[c[0]]}_T{c[1]}_H{c[2]}_I{c[3]}_E{c[4]}_k{c[5]}_sh{int(c[6])}_{c[7]}"


@pytest.mark.parametrize("case", SMALL, ids=_small_id)
def test_small_layers(ora, case):
    dtype, T, H, I, E, k, shared, logits, family = case
    I_sh = (I // 2 if dtype == synth.F32 else 32 * max(1, I // 64)) if shared else 0
    kind = moe.moe_grouped_ffn_kind(T, k, E, H, I, I_sh, dtype)
    assert kind == {"S": moe.MOE_FFN_WEIGHT_STREAM, "G": moe.MOE_FFN_GROUPED_GEMM}[family]
    lay = synth.small_layer(dtype, T, H, I, E, k, seed=500 + T, shared=shared, I_shared=I_sh, logits=logits)
    log(f"small layer {_small_id(case)} kind={kind}")
    b, *_ = run_resident_layer(lay)
    ref = _check_layer(ora, lay, b)
    counts = np.bincount(ref["ids"].ravel(), minlength=E)
    log(f"  tokens per expert {sorted(counts.tolist())}")


# (T, k, H, shared): the combine requests its pairs in groups of 8, so k covers one
# pair, a part group, exactly one group, one more than a group, several groups with a
# part group at the end, and the largest k the library takes.
COMBINE_CASES = [(3, 1, 256, False), (5, 7, 512, True), (4, 8, 2048, False), (6, 9, 1024, True),
                 (2, 20, 4096, True), (3, 32, 256, False)]


@pytest.mark.parametrize("T,k,H,shared", COMBINE_CASES, ids=lambda v: str(v))
def test_combine_pair_groups(ora, T, k, H, shared):
    """y[t] = sum_j w[t][j] * rows[inv[t*k+j]] (+ shared[t]) over whole and part groups of
    pairs, with about a tenth of the pairs dropped (inv = -1, as for expert ids out of
    range), against the oracle's combine of the same rows; the bf16 output is the
    round-to-nearest-even of the f32 one."""
    g = np.random.default_rng(7000 + T * 100 + k)
    n = T * k
    out_rows = g.standard_normal((n, H)).astype(np.float32)
    w = g.random((T, k)).astype(np.float32)
    inv = g.permutation(n).astype(np.int32)
    inv[g.random(n) < 0.1] = -1
    sh = g.standard_normal((T, H)).astype(np.float32) if shared else None
    rows_ref = np.zeros((n, H))
    rows_ref[inv >= 0] = out_rows[inv[inv >= 0]]
    y_ref = ora.combine(rows_ref, w, sh)
    y32 = torch.empty((T, H), dtype=torch.float32, device=dev())
    y16 = torch.empty((T, H), dtype=torch.bfloat16, device=dev())
    args = (to_dev(out_rows), to_dev(w), to_dev(inv), to_dev(sh) if shared else None)
    moe.moe_combine(*args, y32, moe.MOE_F32)
    moe.moe_combine(*args, y16, moe.MOE_BF16)
    torch.cuda.synchronize()
    got = y32.cpu().numpy().astype(np.float64)
    # f32 multiply-adds in a fixed order: each output within (k + 2) units of f32
    # rounding of the sum of the magnitudes it adds up
    mag = np.abs(w.astype(np.float64)[:, :, None] * rows_ref.reshape(T, k, H)).sum(axis=1)
    if shared:
        mag += np.abs(sh)
    bound = (k + 2) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(got - y_ref)
    log(f"combine T={T} k={k} H={H} shared={shared}: max err / bound = {float((err / bound).max()):.3f}")
    assert (err <= bound).all(), f"max err / bound {float((err / bound).max())}"
    np.testing.assert_array_equal(bf16_to_f64(y16), bf16_rne(got))


def test_decode_bf16_full_shape(ora):
    """Decode layer, bf16: H=2048, I=512, 256 experts + 1 shared, top-8; T = 1, 4, 16."""
    c = synth.CONFIGS["decode_bf16"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    pool = synth.torch_bf16_expert_pool(E + 1, H, I, seed=c["seed"], device=dev())
    experts_host = pool.cpu().numpy()
    slots = pool[:E]
    shared = pool[E]
    stride = pool.shape[1]
    for T in c["T_list"]:
        log(f"decode bf16 full T={T}")
        x = synth.encode_activations(synth.BF16, synth.normal_x(c["seed"], T, H, T))
        logits = synth.normal_logits(c["seed"], T, E, T)
        b = L.LayerBuffers(T, E, k, H, I, synth.BF16, I_shared=I)
        L.forward(b, to_dev(logits), to_dev(x), slots, stride, L.identity_slots(E), shared)
        torch.cuda.synchronize()
        lay = dict(dtype=synth.BF16, H=H, I=I, k=k, experts=experts_host[:E], x=x, logits=logits,
                   shared=experts_host[E], I_shared=I)
        _check_layer(ora, lay, b)


def test_decode_mxfp4_full_shape_sampled(ora):
    """Decode layer, MXFP4: H=4096, I=2048, 256 experts, top-6, Zipf-skewed logits;
    T = 1, 8, 64.  Routing and permutation are checked in full, expert outputs and
    y on a sample of tokens."""
    c = synth.CONFIGS["decode_mxfp4"]
    H, I, E, k = c["H"], c["I"], c["E"], c["k"]
    pool = synth.torch_mxfp4_expert_pool(E, H, I, seed=c["seed"], device=dev())
    stride = pool.shape[1]
    for T in c["T_list"]:
        log(f"decode mxfp4 full T={T}")
        x = synth.encode_activations(synth.MXFP4, synth.normal_x(c["seed"], T, H, T))
        logits = synth.zipf_noise_logits(c["seed"], T, E, layer=T % 43, s=c["zipf_s"])
        b = L.LayerBuffers(T, E, k, H, I, synth.MXFP4)
        L.forward(b, to_dev(logits), to_dev(x), pool, stride, L.identity_slots(E))
        torch.cuda.synchronize()
        ids, _, w64 = ora.route_topk(logits, k)
        np.testing.assert_array_equal(b.topk_ids.cpu().numpy(), ids)
        rc, ro, rs, ri = ora.permute(ids, E)
        np.testing.assert_array_equal(b.sorted_rows.cpu().numpy()[: T * k], rs)
        sample = sorted(set([0, T - 1] + list(np.random.default_rng(T).choice(T, size=min(T, 3), replace=False))))
        out_rows = b.out_rows.cpu().numpy().astype(np.float64)
        y_gpu = combine_f32(b, False)
        # one oracle pass per distinct expert over its sampled tokens
        by_expert = {}
        for t in sample:
            for j in range(k):
                by_expert.setdefault(int(ids[t, j]), []).append(t)
        o_ref = {}
        for e, toks in by_expert.items():
            o = ora.expert_rows(synth.MXFP4, pool[e].cpu().numpy(), H, I, x, toks)
            for t, row in zip(toks, o):
                o_ref[(t, e)] = row
        y_ref, y_got, rows_ref, rows_got = [], [], [], []
        for t in sample:
            yt = np.zeros(H)
            for j in range(k):
                o = o_ref[(t, int(ids[t, j]))]
                rows_ref.append(o)
                rows_got.append(out_rows[ri[t * k + j]])
                yt += w64[t, j] * o
            y_ref.append(yt)
            y_got.append(y_gpu[t])
        assert_close_rel(np.array(rows_got), np.array(rows_ref), BF16_REL, "sampled expert rows")
        assert_close_rel(np.array(y_got), np.array(y_ref), BF16_REL, "sampled y")


def test_prefill_mxfp4_full_shape_sampled(ora):
    """Prefill layer, MXFP4: H=4096, I=2048, 256 experts, top-6, T=4096 tokens with
    N(0,1) logits (about 96 +- 10 tokens per expert, every expert active), through
    the grouped GEMM kernels.  Routing and permutation are checked in full; every
    output row of one expert per token-count class (49-64, 65-80, 81-96, 97-112,
    113-128 tokens: 4 to 8 tiles of 16 tokens, 2 to 4 tiles of 32), and y of 8
    tokens, against the oracle element by element."""
    c = synth.CONFIGS["prefill_mxfp4"]
    H, I, E, k, T = c["H"], c["I"], c["E"], c["k"], c["T"]
    assert moe.moe_grouped_ffn_kind(T, k, E, H, I, 0, synth.MXFP4) == moe.MOE_FFN_GROUPED_GEMM
    pool = synth.torch_mxfp4_expert_pool(E, H, I, seed=c["seed"], device=dev())
    stride = pool.shape[1]
    x = synth.encode_activations(synth.MXFP4, synth.normal_x(c["seed"], T, H, 0))
    logits = synth.normal_logits(c["seed"], T, E, 0)
    log(f"prefill mxfp4 full T={T}")
    b = L.LayerBuffers(T, E, k, H, I, synth.MXFP4)
    L.forward(b, to_dev(logits), to_dev(x), pool, stride, L.identity_slots(E))
    torch.cuda.synchronize()
    ids, _, w64 = ora.route_topk(logits, k)
    np.testing.assert_array_equal(b.topk_ids.cpu().numpy(), ids)
    rc, ro, rs, ri = ora.permute(ids, E)
    np.testing.assert_array_equal(b.counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(b.offsets.cpu().numpy(), ro)
    np.testing.assert_array_equal(b.sorted_rows.cpu().numpy()[: T * k], rs)
    np.testing.assert_array_equal(b.inv_rows.cpu().numpy()[: T * k], ri)
    out_rows = b.out_rows.cpu().numpy().astype(np.float64)
    # one expert per token-count class, every one of its rows
    chosen = []
    for lo, hi in ((49, 64), (65, 80), (81, 96), (97, 112), (113, 128)):
        cand = [e for e in range(E) if lo <= rc[e] <= hi]
        if cand:
            chosen.append(cand[len(cand) // 2])
    assert len(chosen) >= 4, f"token counts {sorted(rc.tolist())} miss the classes"
    for e in chosen:
        toks = [int(r) // k for r in rs[ro[e]:ro[e + 1]]]
        log(f"  expert {e}: {len(toks)} tokens")
        ref = ora.expert_rows(synth.MXFP4, pool[e].cpu().numpy(), H, I, x, toks)
        assert_close_rel(out_rows[ro[e]:ro[e + 1]], ref, BF16_REL, f"expert {e} rows ({len(toks)} tokens)")
    # y of 8 tokens (all six experts of each)
    y_gpu = combine_f32(b, False)
    y_bf16 = bf16_to_f64(b.y)
    sample = sorted(set([0, T - 1] + list(np.random.default_rng(7).choice(T, size=6, replace=False))))
    by_expert = {}
    for t in sample:
        for j in range(k):
            by_expert.setdefault(int(ids[t, j]), []).append(t)
    o_ref = {}
    for e, toks in by_expert.items():
        for t, row in zip(toks, ora.expert_rows(synth.MXFP4, pool[e].cpu().numpy(), H, I, x, toks)):
            o_ref[(t, e)] = row
    y_ref = np.array([sum(w64[t, j] * o_ref[(t, int(ids[t, j]))] for j in range(k)) for t in sample])
    r32 = assert_close_rel(y_gpu[sample], y_ref, BF16_REL, "sampled y (f32 output)")
    r16 = assert_close_bf16_output(y_bf16[sample], y_ref, BF16_REL, "sampled y (bf16 output)")
    log(f"  sampled y: max err / RMS = {r32:.2e} (f32 output), {r16:.2e} (bf16 output beyond its half-ulp)")


def test_deterministic_and_doubling_invariant():
    """Same inputs -> bitwise-equal output; doubling every down-projection weight
    (bf16: x2 is exact; MXFP4: every W2 scale +1) doubles y bit for bit."""
    for dtype in (synth.BF16, synth.MXFP4):
        log(f"determinism/doubling dtype={dtype}")
        T, H, I, E, k = 24, 256, 128, 16, 4
        lay = synth.small_layer(dtype, T, H, I, E, k, seed=31, shared=True, I_shared=128)
        b1, *_ = run_resident_layer(lay)
        y1 = b1.y.clone()
        b2, *_ = run_resident_layer(lay)
        assert torch.equal(y1.view(torch.int16), b2.y.view(torch.int16))
        doubled = lay["experts"].copy()
        sh = lay["shared"].copy()
        if dtype == synth.BF16:
            off = synth.slot_offsets(dtype, H, I)["w2"]
            for arr in (doubled[:, off:], sh[None, off:]):
                v = arr.view(np.uint16).astype(np.uint32)
                f = (v << 16).view(np.float32) * 2
                arr[...] = (f.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8).reshape(arr.shape)
        else:
            off = synth.slot_offsets(dtype, H, I)["s2"]
            doubled[:, off:] += 1
            sh[off:] += 1
        b3, *_ = run_resident_layer(dict(lay, experts=doubled, shared=sh))
        y3 = b3.y.float()
        assert torch.equal(y3, 2 * y1.float())


def test_identical_experts_reduce_to_dense_ffn(ora):
    """All experts identical: y = FFN(x) whatever the routing (gate weights sum to 1)."""
    T, H, I, E, k = 12, 256, 128, 8, 3
    lay = synth.small_layer(synth.BF16, T, H, I, E, k, seed=41)
    lay["experts"] = np.stack([lay["experts"][0]] * E)
    b, *_ = run_resident_layer(lay)
    dense = ora.expert_rows(synth.BF16, lay["experts"][0], H, I, lay["x"], list(range(T)))
    check_bf16_output(b, False, dense, BF16_REL, "dense reduction")


def test_empty_batch_and_single_expert():
    log("T=0 and E=1 layers")
    b = L.LayerBuffers(0, 8, 2, 64, 32, synth.BF16)
    pool = torch.zeros((8, moe.moe_expert_bytes(1, 64, 32)), dtype=torch.uint8, device=dev())
    L.forward(b, torch.empty((0, 8), device=dev()), torch.empty((0, 64), dtype=torch.int16, device=dev()), pool,
              pool.shape[1], L.identity_slots(8))
    torch.cuda.synchronize()
    lay = synth.small_layer(synth.BF16, 20, 64, 32, 1, 1, seed=7)
    b1, *_ = run_resident_layer(lay)
    assert torch.all(b1.counts == 20) and torch.all(b1.topk_w == 1.0)
