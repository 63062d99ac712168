"""GPU parity of the batched weight-only product (gptq_dequant_matmul) against the float64
oracle (oracle.dequant_matvec), through the C ABI.

Tolerance: the fp16 products x * (code - z) are exact in float32; within a group of g columns
the matrix cores add them into a float32 sum (at most g additions), which is then scaled (one
rounding) and added to the row's float32 total (d_col / g additions).  Each rounding is at
most 2^-24 of a running magnitude bounded by sum_c |x_c W^_rc|, so the test allows
2^-24 (g + d_col / g + 4) sum_c |x_c W^_rc| per output, g = d_col for per-channel layers.
"""

import numpy as np
import pytest

import oracle as O
from post_weight_quantization_24_amd import gptq as G
from tests.test_gpu_matvec import _torch, acts, packed_layer, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,d_row,d_col,bits,group", [
    (1, 256, 4096, 4, 128),       # one row: tiles mostly empty
    (300, 4096, 4096, 4, 128),    # ragged token tile
    (1000, 1100, 4096, 3, 64),    # INT3 words straddling, ragged output tile
    (5000, 640, 1024, 2, 16),     # one-MFMA groups
    (77, 96, 8192, 8, 0),         # per-channel, fewer outputs than a tile
    (130, 200, 96, 4, 32),        # d_col with a half K stage
    (2500, 300, 2048, 2, 128),    # INT2 read packed, ragged tiles both ways
    (129, 257, 640, 4, 0),        # per-channel INT4 read packed, one row past a tile each way
    (64, 512, 1024, 8, 256),      # INT8 read packed, groups of four stages
    (200, 384, 1536, 4, 256),     # INT4 128-column stages, groups of two
    (100, 300, 1600, 4, 64),      # INT4 with 64-column groups: 64-column stages
    (70, 260, 192, 4, 0),         # per-channel INT4, d_col not a multiple of 128
])
def test_dequant_matmul(n, d_row, d_col, bits, group):
    torch = _torch()
    say("dequant_matmul", n, d_row, d_col, bits, group)
    rng = np.random.default_rng(1020 + d_col + bits)
    words, scales, zeros = packed_layer(rng, d_row, d_col, bits, group)
    x = acts(rng, n, d_col)
    dev = "cuda:0"
    y = G.dequant_matmul(torch.from_numpy(words.view(np.int32)).to(dev),
                         torch.from_numpy(scales).to(dev), torch.from_numpy(zeros).to(dev),
                         torch.from_numpy(x).to(dev), bits, group, d_col)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    ref = O.dequant_matvec(words, scales, zeros, bits, group, d_col, x)
    g = d_col if group == 0 else group
    Wh = O.dequantize(O.unpack_codes(words, bits, d_col), scales, zeros, g)
    tol = 2.0 ** -24 * (g + d_col / g + 4) * (np.abs(x.astype(np.float64)) @ np.abs(Wh).T)
    err = np.abs(got - ref)
    say("max err / tol %.3g" % float((err / tol).max()))
    assert np.all(err <= tol)


def test_dequant_matmul_matches_matvec():
    """The small-n path and the matrix-core path compute the same product."""
    torch = _torch()
    say("dequant_matmul against dequant_matvec")
    rng = np.random.default_rng(1030)
    d_row, d_col, bits, group, n = 2048, 4096, 4, 128, 64
    words, scales, zeros = packed_layer(rng, d_row, d_col, bits, group)
    dev = "cuda:0"
    q = torch.from_numpy(words.view(np.int32)).to(dev)
    s = torch.from_numpy(scales).to(dev)
    z = torch.from_numpy(zeros).to(dev)
    x = torch.from_numpy(acts(rng, n, d_col)).to(dev)
    a = G.dequant_matmul(q, s, z, x, bits, group, d_col)
    b = G.dequant_matvec(q, s, z, x, bits, group, d_col)
    torch.cuda.synchronize()
    Wh = O.dequantize(O.unpack_codes(words, bits, d_col), scales, zeros, group)
    mag = np.abs(x.cpu().numpy().astype(np.float64)) @ np.abs(Wh).T
    # the sum of the two paths' bounds (this file's and the small-n test's)
    tol = 2.0 ** -24 * ((group + d_col / group + 4) + (32 + d_col / 32 + 6)) * mag
    err = (a - b).abs().cpu().numpy()
    say("max difference / bound %.3g" % float((err / tol).max()))
    assert np.all(err <= tol)


@pytest.mark.slow
def test_dequant_matmul_70b_shape_sampled():
    """The bench's batched case (gate_proj 28672 x 8192 INT4 g128 at 2048 rows, the launch
    configuration bench.py times) on sampled outputs, each computed by the oracle from its
    row of codes and its activation row."""
    torch = _torch()
    say("dequant_matmul 70B shape, sampled")
    d_row, d_col, bits, group, n = 28672, 8192, 4, 128, 2048
    rng = np.random.default_rng(1040)
    # uniformly random words are uniformly random 4-bit codes (as the bench draws them)
    words = rng.integers(0, 1 << 32, (d_row, d_col * bits // 32), dtype=np.uint64).astype(np.uint32)
    scales = rng.uniform(0.002, 0.02, (d_row, d_col // group)).astype(np.float32)
    zeros = rng.integers(0, 1 << bits, (d_row, d_col // group)).astype(np.uint8)
    x = acts(rng, n, d_col)
    dev = "cuda:0"
    y = G.dequant_matmul(torch.from_numpy(words.view(np.int32)).to(dev),
                         torch.from_numpy(scales).to(dev), torch.from_numpy(zeros).to(dev),
                         torch.from_numpy(x).to(dev), bits, group, d_col)
    torch.cuda.synchronize()
    rows = rng.integers(0, d_row, 64)
    toks = rng.integers(0, n, 64)
    got = y[torch.from_numpy(toks).to(dev), torch.from_numpy(rows).to(dev)].cpu().numpy()
    worst = 0.0
    for t, r, v in zip(toks, rows, got):
        ref = O.dequant_matvec(words[r:r + 1], scales[r:r + 1], zeros[r:r + 1], bits, group, d_col,
                               x[t:t + 1])[0, 0]
        wh = O.dequantize(O.unpack_codes(words[r:r + 1], bits, d_col), scales[r:r + 1],
                          zeros[r:r + 1], group)[0]
        tol = 2.0 ** -24 * (group + d_col / group + 4) * float(np.abs(x[t].astype(np.float64)) @ np.abs(wh))
        worst = max(worst, abs(float(v) - ref) / tol)
        assert abs(float(v) - ref) <= tol, (t, r)
    say("max err / tol over 64 samples %.3g" % worst)


def test_dequant_matmul_strided_x():
    """x with a row stride above d_col (a column slice of a wider activation buffer), on the
    packed path; the product equals the one on a contiguous copy bit for bit."""
    torch = _torch()
    say("dequant_matmul strided x")
    rng = np.random.default_rng(1031)
    d_row, d_col, bits, group, n = 700, 1024, 4, 128, 333
    words, scales, zeros = packed_layer(rng, d_row, d_col, bits, group)
    dev = "cuda:0"
    q = torch.from_numpy(words.view(np.int32)).to(dev)
    s = torch.from_numpy(scales).to(dev)
    z = torch.from_numpy(zeros).to(dev)
    wide = torch.from_numpy(acts(rng, n, d_col + 64)).to(dev)
    xs = wide[:, 32:32 + d_col]
    assert xs.stride(0) == d_col + 64
    a = G.dequant_matmul(q, s, z, xs, bits, group, d_col)
    b = G.dequant_matmul(q, s, z, xs.contiguous(), bits, group, d_col)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
