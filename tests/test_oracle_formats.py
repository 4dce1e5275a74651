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


def test_mxfp4_slot_layout_hand_built(ora):
    """A slot assembled byte by byte from the documented layout decodes as intended.

    H = I = 32: W13 codes [64][16] bytes, W2 codes [32][16], W13 scales [64][1], W2 scales [32][1].
    """
    H = I = 32
    nbytes = ora.expert_bytes(ora.MXFP4, H, I)
    assert nbytes == 3 * H * I // 2 + 3 * H * I // 32
    slot = np.zeros(nbytes, np.uint8)
    w13_codes = 0
    w2_codes = 2 * I * H // 2
    w13_scales = w2_codes + H * I // 2
    w2_scales = w13_scales + 2 * I * H // 32
    assert w2_scales + H * I // 32 == nbytes
    slot[w13_scales:w13_scales + 2 * I] = 127          # scale 1.0 for every W13 row
    slot[w2_scales:w2_scales + H] = 127
    slot[w13_codes + 0] = 0x21                          # gate row 0: elem 0 = code 1 (0.5), elem 1 = code 2 (1.0)
    slot[w13_codes + I * (H // 2) + 3] = 0x9F           # up row 0 (W13 row I), byte 3: elem 6 = code 15 (-6), elem 7 = code 9 (-0.5)
    slot[w13_scales + I] = 129                          # up row 0 scale 4
    slot[w2_codes + 5 * (I // 2) + 15] = 0x70           # down row 5, byte 15: elem 30 = 0, elem 31 = code 7 (6)
    slot[w2_scales + 5] = 126                           # down row 5 scale 0.5
    wg, wu, wd = ora.decode_expert(ora.MXFP4, slot, H, I)
    exp_g = np.zeros((I, H)); exp_g[0, 0] = 0.5; exp_g[0, 1] = 1.0
    exp_u = np.zeros((I, H)); exp_u[0, 6] = -24.0; exp_u[0, 7] = -2.0
    exp_d = np.zeros((H, I)); exp_d[5, 31] = 3.0
    np.testing.assert_array_equal(wg, exp_g)
    np.testing.assert_array_equal(wu, exp_u)
    np.testing.assert_array_equal(wd, exp_d)


@pytest.mark.parametrize("dtype", [0, 1])
def test_dense_slot_layout_hand_built(ora, dtype):
    H, I = 4, 2
    vals = np.arange(3 * H * I, dtype=np.float32) - 7.0  # exactly representable in bf16
    if dtype == 0:
        slot = vals.view(np.uint8)
    else:
        slot = (vals.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8)
    wg, wu, wd = ora.decode_expert(dtype, slot, H, I)
    np.testing.assert_array_equal(wg, vals[:I * H].reshape(I, H))
    np.testing.assert_array_equal(wu, vals[I * H:2 * I * H].reshape(I, H))
    np.testing.assert_array_equal(wd, vals[2 * I * H:].reshape(H, I))


def test_mxfp4_roundtrip_of_representable_values(ora):
    """Values c * 2^e with c an E2M1 value and a block max of 6 * 2^e survive the
    generator's encoding and the oracle's decoding exactly."""
    g = np.random.default_rng(3)
    H, I = 64, 32
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
