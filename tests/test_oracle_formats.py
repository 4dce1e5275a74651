"""Pins of the oracle's format decoders against the format definitions.

The oracle decodes with lookup tables and bit tricks; these tests derive the same
values from the bit-field definitions and from library routines instead.
"""
import math
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_from_fields(code):
    # 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; exponent 0 is subnormal.
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m * 0.5)
    return -mag if s else mag


def test_e2m1_all_codes_match_bitfield_definition(ora):
    for code in range(16):
        assert ora.e2m1_value(code) == _e2m1_from_fields(code)


def test_e2m1_matches_spec_table(ora):
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for c, v in rows:
        got = ora.e2m1_value(int(c))
        assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v))


def test_e8m0_all_codes(ora):
    for c in range(255):
        assert ora.e8m0_value(c) == math.ldexp(1.0, c - 127)
    assert math.isnan(ora.e8m0_value(255))


def test_bf16_widening_matches_numpy(ora):
    g = np.random.default_rng(0)
    bits = g.integers(0, 1 << 16, size=4000, dtype=np.uint32).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    for b, r in zip(bits, ref):
        if np.isnan(r):
            continue
        assert ora.bf16_value(int(b)) == float(r)


def _frag(row, k, K, KS):
    """Fragment index of element (row, k) in the tiled layout, written out from its
    description: 16-row x KS-column tiles, row-tile major then column step, 64
    fragments per tile ordered by 16*group + row%16, group = (k%KS)//(KS/4)."""
    nk = -(-K // KS)
    return ((row // 16) * nk + k // KS) * 64 + 16 * ((k % KS) // (KS // 4)) + row % 16


def _scale_pos(row, k, K):
    """Byte of the scale of MXFP4 element (row, k), written out from the layout
    description: per row tile, 1 KB blocks of 16 column steps; fragment f owns 16
    bytes of a block, byte i being its scale at step 16*block + i."""
    nk = -(-K // 128)
    nblocks = -(-nk // 16)
    step = k // 128
    f = 16 * ((k % 128) // 32) + row % 16
    return ((row // 16) * nblocks + step // 16) * 1024 + 16 * f + step % 16


def test_mxfp4_slot_layout_hand_built(ora):
    """A slot assembled byte by byte from the layout description decodes as intended.

    H = I = 32: W13 has 64 stored rows (4 tiles x 1 padded step), W2 32 rows (2 tiles);
    codes 4096 + 2048 bytes, scales 4 + 2 blocks of 1 KB.  Stored W13 row 16t+q is
    gate row 8t+q for q < 8, up row 8t+q-8 otherwise.
    """
    H = I = 32
    nbytes = ora.expert_bytes(ora.MXFP4, H, I)
    assert nbytes == 4096 + 2048 + 4096 + 2048
    c13, c2, s13, s2 = 0, 4096, 6144, 10240
    slot = np.zeros(nbytes, np.uint8)
    slot[s13:s13 + 4096] = 127     # scale 1.0 everywhere (padding included)
    slot[s2:s2 + 2048] = 127
    f = _frag(0, 0, H, 128)          # gate row 0 -> stored row 0; elements 0, 1
    slot[c13 + 16 * f] = 0x21        # elem 0 = code 1 (0.5), elem 1 = code 2 (1.0)
    f = _frag(8, 6, H, 128)          # up row 0 -> stored row 8; elements 6, 7 in byte 3
    slot[c13 + 16 * f + 3] = 0x9F    # elem 6 = code 15 (-6), elem 7 = code 9 (-0.5)
    slot[s13 + _scale_pos(8, 6, H)] = 129   # scale 4
    f = _frag(16 + 1, 5, H, 128)     # gate row 9 -> stored row 17; element 5 = high nibble of byte 2
    slot[c13 + 16 * f + 2] = 0x50    # code 5 (3.0)
    f = _frag(5, 31, I, 128)         # down row 5, element 31 = high nibble of byte 15
    slot[c2 + 16 * f + 15] = 0x70    # code 7 (6.0)
    slot[s2 + _scale_pos(5, 31, I)] = 126   # scale 0.5
    wg, wu, wd = ora.decode_expert(ora.MXFP4, slot, H, I)
    exp_g = np.zeros((I, H)); exp_g[0, 0] = 0.5; exp_g[0, 1] = 1.0; exp_g[9, 5] = 3.0
    exp_u = np.zeros((I, H)); exp_u[0, 6] = -24.0; exp_u[0, 7] = -2.0
    exp_d = np.zeros((H, I)); exp_d[5, 31] = 3.0
    np.testing.assert_array_equal(wg, exp_g)
    np.testing.assert_array_equal(wu, exp_u)
    np.testing.assert_array_equal(wd, exp_d)


def test_bf16_slot_layout_hand_built(ora):
    H, I = 64, 32
    g = np.random.default_rng(4)
    wg = g.integers(-50, 50, size=(I, H)).astype(np.float32) / 8   # exactly representable in bf16
    wu = g.integers(-50, 50, size=(I, H)).astype(np.float32) / 8
    wd = g.integers(-50, 50, size=(H, I)).astype(np.float32) / 8
    bits = lambda v: int(np.float32(v).view(np.uint32) >> 16)
    w13_bytes = 2 * 2 * I * H
    slot = np.zeros(w13_bytes + 2 * H * I, np.uint8)
    u16 = slot.view(np.uint16)
    for j in range(I):
        for k in range(H):
            for row, val in ((16 * (j // 8) + j % 8, wg[j, k]), (16 * (j // 8) + 8 + j % 8, wu[j, k])):
                u16[(16 * _frag(row, k, H, 32)) // 2 + k % 8] = bits(val)
    for r in range(H):
        for k in range(I):
            u16[(w13_bytes + 16 * _frag(r, k, I, 32)) // 2 + k % 8] = bits(wd[r, k])
    dg, du, dd = ora.decode_expert(ora.BF16, slot, H, I)
    np.testing.assert_array_equal(dg, wg)
    np.testing.assert_array_equal(du, wu)
    np.testing.assert_array_equal(dd, wd)
    # the generator's packing agrees byte for byte
    np.testing.assert_array_equal(synth.pack_expert(synth.BF16, wg, wu, wd), slot)


def test_f32_slot_layout_hand_built(ora):
    H, I = 4, 2
    vals = np.arange(3 * H * I, dtype=np.float32) - 7.0
    wg, wu, wd = ora.decode_expert(ora.F32, vals.view(np.uint8), H, I)
    np.testing.assert_array_equal(wg, vals[:I * H].reshape(I, H))
    np.testing.assert_array_equal(wu, vals[I * H:2 * I * H].reshape(I, H))
    np.testing.assert_array_equal(wd, vals[2 * I * H:].reshape(H, I))


def test_mxfp4_padding_for_k_not_multiple_of_128(ora):
    H, I = 160, 96   # K = 160 -> 2 steps (96 padded columns); K = 96 -> 1 step (32 padded)
    nb = ora.expert_bytes(ora.MXFP4, H, I)
    # codes: 2 steps and 1 step of 1 KB per row tile; scales: one 1 KB block per row tile
    assert nb == (2 * I // 16) * 2 * 1024 + (H // 16) * 1 * 1024 + (2 * I // 16) * 1024 + (H // 16) * 1024
    assert nb == synth.expert_bytes(synth.MXFP4, H, I)


def test_mxfp4_scales_past_sixteen_steps(ora):
    """K = 17 * 128: each row tile holds two scale blocks, the second with one used
    step; a scale written at step 16 (block 1, byte 0) and one at step 15 (block 0,
    byte 15) land on their own elements only."""
    H, I = 17 * 128, 32
    nb = ora.expert_bytes(ora.MXFP4, H, I)
    c13 = 0
    s13 = (2 * I // 16) * 17 * 1024 + (H // 16) * 1 * 1024
    assert nb == s13 + (2 * I // 16) * 2 * 1024 + (H // 16) * 1024
    slot = np.zeros(nb, np.uint8)
    slot[s13:] = 127
    for row, k, code, sc in ((0, 16 * 128 + 3, 0x02, 130), (3, 15 * 128 + 64, 0x01, 125)):
        f = _frag(row, k, H, 128)
        e = k % 32
        slot[c13 + 16 * f + e // 2] |= code << (4 * (e % 2))
        slot[s13 + _scale_pos(row, k, H)] = sc
    wg, wu, wd = ora.decode_expert(ora.MXFP4, slot, H, I)
    exp_g = np.zeros((I, H))
    exp_g[0, 16 * 128 + 3] = 1.0 * 8.0     # code 2 (1.0) x 2^3
    exp_g[3, 15 * 128 + 64] = 0.5 * 0.25   # code 1 (0.5) x 2^-2
    np.testing.assert_array_equal(wg, exp_g)
    np.testing.assert_array_equal(wu, np.zeros((I, H)))
    np.testing.assert_array_equal(wd, np.zeros((H, I)))


def test_mxfp4_roundtrip_of_representable_values(ora):
    """Values c * 2^e with c an E2M1 value and a block max of 6 * 2^e survive the
    generator's encoding and the oracle's decoding exactly."""
    g = np.random.default_rng(3)
    H, I = 17 * 128, 96   # W13 rows span two scale blocks (the second partly padding)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])

    def mat(rows, K):
        m = g.choice(mags, size=(rows, K)) * g.choice([-1, 1], size=(rows, K))
        m = m.reshape(rows, K // 32, 32)
        m[:, :, 0] = 6.0  # pin each block's max so the shared exponent is e
        e = g.integers(-12, 3, size=(rows, K // 32, 1))
        return (m * np.ldexp(1.0, e)).reshape(rows, K)

    wg, wu, wd = mat(I, H), mat(I, H), mat(H, I)
    slot = synth.pack_expert(synth.MXFP4, wg, wu, wd)
    dg, du, dd = ora.decode_expert(ora.MXFP4, slot, H, I)
    np.testing.assert_array_equal(dg, wg)
    np.testing.assert_array_equal(du, wu)
    np.testing.assert_array_equal(dd, wd)


# ---- MXFP8 (E4M3) activations of the native FP4 path (OCP MX v1.0) -------------

def _e4m3_formula(v):
    """E4M3 code of v by the closed-form rounding (not the oracle's search): RNE in
    the subnormal steps of 2^-9 below 2^-6, else RNE of the 3-bit mantissa at
    v's own exponent; beyond 448 the largest finite value."""
    import math
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a < 2.0 ** -6:
        return sign | int(round(a * 512))          # Python round(): ties to even
    _, e2 = math.frexp(a)
    e = e2 - 1
    m = int(round(math.ldexp(a, 3 - e)))           # 8 .. 16
    if m == 16:
        e, m = e + 1, 8
    if e > 8 or (e == 8 and m > 14):
        return sign | 0x7E
    return sign | ((e + 7) << 3) | (m - 8)


def test_e4m3_values_from_the_spec(ora):
    import math
    assert ora.e4m3_value(0x7E) == 448.0               # largest finite
    assert ora.e4m3_value(0x08) == 2.0 ** -6           # smallest normal
    assert ora.e4m3_value(0x01) == 2.0 ** -9           # smallest subnormal
    assert ora.e4m3_value(0x38) == 1.0 and ora.e4m3_value(0x39) == 1.125 and ora.e4m3_value(0x36) == 0.875
    assert math.isnan(ora.e4m3_value(0x7F)) and math.isnan(ora.e4m3_value(0xFF))
    vals = [ora.e4m3_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(vals, vals[1:])) and vals[0] == 0.0
    assert all(ora.e4m3_value(c | 0x80) == -ora.e4m3_value(c) for c in range(1, 0x7F))


def test_mx8_quantize_against_closed_form_rounding(ora):
    import math
    g = np.random.default_rng(8)
    blocks = [g.standard_normal(32) * s for s in (1.0, 1e-3, 37.0, 3e-30)]
    # crafted: exact halfway points (ties), the saturation band of the top element,
    # zeros and -0, subnormal steps
    b = np.full(32, 0.0)
    b[0] = 1.0                                           # X = -8: elements scale by 256
    b[1:9] = [(1 + 1 / 16) / 256, (1 + 3 / 16) / 256, (1 + 5 / 16) / 256, 2 ** -9 * 1.5 / 256,
              2 ** -9 * 2.5 / 256, -(1 + 1 / 16) / 256, -0.0, 0.0]
    blocks.append(b)
    sat = np.full(32, 0.25)
    sat[0] = 1.99                                        # scaled to ~509.4: clamps to 448
    blocks.append(sat)
    blocks.append(np.zeros(32))
    x = synth.bf16_bits(np.concatenate(blocks).astype(np.float32)).reshape(len(blocks), 32)
    codes, scales = ora.mx8_quantize(x)
    for r in range(x.shape[0]):
        v = synth.bf16_bits_to_f32(x[r]).astype(np.float64)
        amax = np.abs(v).max()
        X = -127 if amax == 0 else max(-127, math.frexp(amax)[1] - 1 - 8)
        assert scales[r, 0] == X + 127
        for i in range(32):
            assert codes[r, i] == _e4m3_formula(math.ldexp(v[i], -X)), (r, i, v[i])
    assert scales[4, 0] == 127 - 8 and codes[4, 7] == 0x80 and codes[4, 8] == 0x00
    # ties go to the even code: 1.0625 -> 1.0, 1.1875 -> 1.25, 1.5 and 2.5 subnormal steps -> 2
    assert list(codes[4, 1:6]) == [0x38, 0x3A, 0x3A, 0x02, 0x02] and codes[4, 6] == 0xB8
    assert codes[5, 0] == 0x7E and scales[6, 0] == 0


def test_mx8_quantize_is_identity_on_representable_values(ora):
    """Values already of the form E4M3 x 2^X (block maximum fixing X) come back
    unchanged, so an A8 layer on such activations equals the MXFP4 layer exactly."""
    g = np.random.default_rng(9)
    T, H = 3, 128
    codes = g.integers(0, 0x7F, size=(T, H)).astype(np.uint8) | (g.integers(0, 2, size=(T, H)) * 0x80).astype(np.uint8)
    codes[:, ::32] = 0x7E                                  # block maximum 448 -> X fixed by the exponent below
    X = g.integers(-20, 20, size=(T, H // 32))
    vals = np.array([[ora.e4m3_value(int(c)) for c in row] for row in codes]) * np.repeat(2.0 ** X, 32, axis=1)
    x = synth.bf16_bits(vals.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(x).astype(np.float64), vals)   # representable in bf16 too
    q, s = ora.mx8_quantize(x)
    np.testing.assert_array_equal(q, codes)
    np.testing.assert_array_equal(s.astype(int), X + 127)
    H2, I, E, k = 128, 64, 4, 2
    lay = synth.small_layer(synth.MXFP4, T, H2, I, E, k, seed=3)
    a = ora.layer(synth.MXFP4, lay["experts"], x, lay["logits"], k, H2, I)
    b = ora.layer(ora.MXFP4_A8, lay["experts"], x, lay["logits"], k, H2, I)
    np.testing.assert_array_equal(a["y"], b["y"])
