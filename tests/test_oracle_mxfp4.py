"""Pins of the oracle's MXFP4 expert weights (dequantize_mxfp4, decode_fp4_e2m1,
decode_e8m0) against facts fixed outside it:

  * the FP4 E2M1 element values the OCP Microscaling (MX) v1.0 specification
    lists for the format (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; the sign in
    bit 3), and its E8M0 scale values (2^(s - 127), 255 = NaN);
  * hand-packed bytes with hand-computed values (nibble order, scale groups);
  * the INT4 dequantiser (pinned by tests/test_oracle_pins.py): weights whose
    values both formats can hold must dequantise, and run through the layer,
    identically.
"""
import numpy as np
import pytest

import oracle

# value of each 4-bit code, as the specification's table gives it
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_code_values():
    got = oracle.decode_fp4_e2m1(np.arange(16))
    assert got.tolist() == E2M1_TABLE
    assert np.signbit(got[8]) and not np.signbit(got[0])  # code 8 is -0


def test_e8m0_values():
    got = oracle.decode_e8m0(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert got[0] == 2.0 ** -127 and got[1] == 2.0 ** -126
    assert got[2] == 0.5 and got[3] == 1.0 and got[4] == 2.0
    assert got[5] == 2.0 ** 127
    assert np.isnan(got[6])


def test_hand_packed_row():
    # one row of 64 channels = 2 groups; byte i holds channel 2i (low nibble) and 2i+1 (high)
    q = np.zeros((1, 32), np.uint8)
    q[0, 0] = 0x21   # ch0 = code 1 (0.5), ch1 = code 2 (1.0)
    q[0, 1] = 0xF7   # ch2 = code 7 (6.0), ch3 = code 15 (-6.0)
    q[0, 15] = 0x9C  # ch30 = code 12 (-2.0), ch31 = code 9 (-0.5)
    q[0, 16] = 0x35  # ch32 = code 5 (3.0), ch33 = code 3 (1.5)  (group 1)
    s = np.array([[126, 130]], np.uint8)  # group 0: 0.5, group 1: 8
    W = oracle.dequantize_mxfp4(q, s)
    expect = np.zeros((1, 64))
    expect[0, [0, 1, 2, 3, 30, 31]] = [0.25, 0.5, 3.0, -3.0, -1.0, -0.25]
    expect[0, [32, 33]] = [24.0, 12.0]
    assert np.array_equal(W, expect)


# codes of the values both formats hold
_VAL_TO_CODE = {0: 0, 1: 2, 2: 4, 3: 5, 4: 6, 6: 7, -1: 10, -2: 12, -3: 13, -4: 14, -6: 15}


def _same_matrix(rng, N, K, scale_exp):
    vals = rng.choice(list(_VAL_TO_CODE), size=(N, K))
    u = (vals + 8).astype(np.uint8)                           # INT4 nibble: q + 8
    c = np.vectorize(_VAL_TO_CODE.get)(vals).astype(np.uint8)  # FP4 code
    q4 = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    f4 = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    G = K // 32
    e = rng.choice(scale_exp, size=(N, G))
    s16 = np.ldexp(1.0, e).astype(np.float16)  # exact powers of two in fp16
    s8 = (127 + e).astype(np.uint8)
    return q4, s16, f4, s8


def test_mxfp4_equals_int4_on_shared_values():
    rng = np.random.default_rng(7)
    q4, s16, f4, s8 = _same_matrix(rng, 48, 256, [-6, -5, -4, 0, 3])
    assert np.array_equal(oracle.dequantize_mxfp4(f4, s8), oracle.dequantize(q4, s16))


def test_mxfp4_layer_equals_int4_layer_on_shared_values():
    rng = np.random.default_rng(11)
    E, H, I, k, M = 4, 128, 64, 2, 5
    experts4, expertsf = {}, {}
    for ex in range(E):
        a = _same_matrix(rng, 2 * I, H, [-6, -5])
        b = _same_matrix(rng, H, I, [-6, -5])
        experts4[ex] = (a[0], a[1], b[0], b[1])
        expertsf[ex] = (a[2], a[3], b[2], b[3])
    c4 = oracle.DequantCache(lambda ex: experts4[ex], fmt="int4")
    cf = oracle.DequantCache(lambda ex: expertsf[ex], fmt="mxfp4")
    x = rng.standard_normal((M, H))
    logits = rng.standard_normal((M, E)).astype(np.float32)
    out4, ids, w = oracle.layer(x, logits, k, c4)
    outf, _, _ = oracle.layer(x, logits, k, cf)
    assert np.array_equal(out4, outf)


@pytest.mark.parametrize("g", [0, 3])
def test_scale_touches_only_its_group(g):
    rng = np.random.default_rng(3)
    q = rng.integers(0, 256, (2, 64), np.uint8)
    s = np.full((2, 4), 127, np.uint8)
    base = oracle.dequantize_mxfp4(q, s)
    s2 = s.copy()
    s2[1, g] = 129  # x4
    W = oracle.dequantize_mxfp4(q, s2)
    cols = slice(32 * g, 32 * g + 32)
    assert np.array_equal(W[1, cols], 4 * base[1, cols])
    mask = np.ones_like(W, bool)
    mask[1, cols] = False
    assert np.array_equal(W[mask], base[mask])
