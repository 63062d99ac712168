"""Pins of the oracle's weight-only quantized product (dequant_matvec), the step after the
quantizer: page "量化", section GPTQ (per-channel INT4 output for single-batch inference) and
section AWQ (W4A16, dequantization inside the matrix product).

Every expected value below is worked out by hand from the packed format (code (r, c) at bits
[c*b, c*b + b) of row r's little-endian bitstream) and the grid s (code - z); the last two
tests tie the product to the pinned loss identity and to the pinned dequantizer.
"""

import numpy as np

import oracle as O


def _w(*words):
    return np.array([list(words)], dtype=np.uint32)


def test_int4_known_word():
    # 0x76543210 holds the codes 0, 1, ..., 7 (nibble c is code c); s = 0.5, z = 3
    # -> W^ = 0.5 * ([0..7] - 3) = [-1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2]
    words = _w(0x76543210)
    s = np.array([[0.5]]); z = np.array([[3]])
    y = O.dequant_matvec(words, s, z, 4, 0, 8, np.ones((1, 8)))
    assert y.shape == (1, 1) and y[0, 0] == 2.0          # sum of W^
    x = np.arange(1, 9, dtype=np.float64)[None, :]
    # -1.5 - 2 - 1.5 + 0 + 2.5 + 6 + 10.5 + 16 = 30
    assert O.dequant_matvec(words, s, z, 4, 0, 8, x)[0, 0] == 30.0


def test_int3_codes_straddling_words():
    # codes c % 8 over 32 columns: each run 0..7 is the 24-bit value 0o76543210 = 0xFAC688;
    # four runs fill 96 bits: 0x88FAC688, 0xC688FAC6, 0xFAC688FA
    words = _w(0x88FAC688, 0xC688FAC6, 0xFAC688FA)
    one = np.ones((1, 32))
    # one group, s = 1, z = 4: 4 runs x (0 + 1 + ... + 7 - 8 * 4) = 4 * (-4) = -16
    assert O.dequant_matvec(words, np.array([[1.0]]), np.array([[4]]), 3, 0, 32, one)[0, 0] == -16
    # groups of 8 (one run each): s = [1, 2, 0.5, 4], z = [4, 0, 7, 3]
    # 1 (28 - 32) + 2 (28 - 0) + 0.5 (28 - 56) + 4 (28 - 24) = -4 + 56 - 14 + 16 = 54
    s = np.array([[1.0, 2.0, 0.5, 4.0]]); z = np.array([[4, 0, 7, 3]])
    assert O.dequant_matvec(words, s, z, 3, 8, 32, one)[0, 0] == 54.0


def test_int2_known_word():
    # 0xE4 = 0b11_10_01_00 holds codes 0, 1, 2, 3; four copies give codes c % 4 over 16 columns
    # s = 0.25, z = 2: W^_c = 0.25 (c % 4 - 2); x_c = c
    # per run k (c = 4k..4k+3): 0.25 (-2 (4k) - (4k + 1) + (4k + 3)) = 0.25 (2 - 8k)
    # sum over k = 0..3: 0.25 (8 - 48) = -10
    words = _w(0xE4E4E4E4)
    x = np.arange(16, dtype=np.float64)[None, :]
    y = O.dequant_matvec(words, np.array([[0.25]]), np.array([[2]]), 2, 0, 16, x)
    assert y[0, 0] == -10.0


def test_product_matches_layer_loss():
    # sum over tokens of ||W x_t - y_t||^2 = ||(W - W^) X^T||^2 = 1/2 sum_r D_r H D_r^T with
    # H = 2 X^T X (the pinned loss identity); a transposed operand or a wrong group fails it
    rng = np.random.default_rng(11)
    d_row, d_col, n, bits, group = 8, 64, 50, 4, 32
    W = rng.standard_normal((d_row, d_col)) * 0.02
    X = rng.standard_normal((n, d_col)) * np.exp(0.5 * rng.standard_normal(d_col))
    q = O.rtn_quantize(W, bits, group, False)
    words = O.pack_codes(q["codes"], bits)
    Y = O.dequant_matvec(words, q["scales"], q["zeros"], bits, group, d_col, X)
    direct = float(np.sum((X @ W.T - Y) ** 2))
    w_hat = O.dequantize(q["codes"], q["scales"], q["zeros"], group)
    via_h = O.layer_loss(W, w_hat, O.hessian(X))
    assert abs(direct - via_h) <= 1e-9 * via_h


def test_unit_vectors_give_columns():
    rng = np.random.default_rng(12)
    d_row, d_col, bits, group = 5, 96, 3, 32
    codes = rng.integers(0, 8, (d_row, d_col))
    s = rng.uniform(0.5, 2.0, (d_row, d_col // group)); z = rng.integers(0, 8, (d_row, d_col // group))
    Y = O.dequant_matvec(O.pack_codes(codes, bits), s, z, bits, group, d_col, np.eye(d_col))
    assert np.array_equal(Y.T, O.dequantize(codes, s, z, group))
