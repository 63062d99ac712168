"""GPU parity of the weight-only quantized product (gptq_dequant_matvec) against the float64
oracle (oracle.dequant_matvec), through the C ABI.

Tolerance: the kernel sums in float32.  Each output is a sum of at most 32 products per run
(accumulated in order), d_col / 32 runs and a 6-level butterfly, so each addition contributes
at most 2^-24 of the running magnitude, which is bounded by sum_c |x_c W^_rc|.  The test
allows 2^-24 * (32 + d_col / 32 + 6) * sum_c |x_c W^_rc| per output.  The fp16 products of
the 4-bit path are exact in float32 (q - z is an integer below 16 in magnitude).
"""

import numpy as np
import pytest

import oracle as O
from post_weight_quantization_24_amd import gptq as G
from post_weight_quantization_24_amd import synth

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch


def say(*a):
    print("[gpu-case]", *a, flush=True)


def packed_layer(rng, d_row, d_col, bits, group):
    g = d_col if group == 0 else group
    codes = rng.integers(0, 1 << bits, (d_row, d_col))
    scales = rng.uniform(0.002, 0.02, (d_row, d_col // g)).astype(np.float32)
    zeros = rng.integers(0, 1 << bits, (d_row, d_col // g)).astype(np.uint8)
    return O.pack_codes(codes, bits), scales, zeros


def acts(rng, n, d_col):
    return (rng.standard_normal((n, d_col)) * np.exp(0.5 * rng.standard_normal(d_col))).astype(np.float16)


def run_gpu(words, scales, zeros, x, bits, group, d_col):
    torch = _torch()
    dev = "cuda:0"
    qw = torch.from_numpy(words.view(np.int32)).to(dev)
    sc = torch.from_numpy(scales).to(dev)
    ze = torch.from_numpy(zeros).to(dev)
    xd = torch.from_numpy(x).to(dev)
    y = G.dequant_matvec(qw, sc, ze, xd, bits, group, d_col)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def check(words, scales, zeros, x, bits, group, d_col, rows=None):
    y = run_gpu(words, scales, zeros, x, bits, group, d_col)
    sel = slice(None) if rows is None else rows
    g = d_col if group == 0 else group
    w_hat = O.dequantize(O.unpack_codes(words[sel], bits, d_col), scales[sel], zeros[sel], g)
    ref = O.dequant_matvec(words[sel], scales[sel], zeros[sel], bits, group, d_col, x)
    bound = np.abs(x.astype(np.float64)) @ np.abs(w_hat).T
    tol = 2.0 ** -24 * (32 + d_col / 32 + 6) * bound
    got = y[:, sel]
    err = np.abs(got - ref)
    say("max err / tol %.3g" % float((err / np.maximum(tol, 1e-300)).max()))
    assert np.all(err <= tol)
    return y


CASES = [  # d_row, d_col, bits, group, n
    (77, 256, 4, 128, 1), (300, 4096, 4, 128, 1), (64, 4096, 4, 0, 3), (129, 1024, 4, 32, 8),
    (100, 1024, 3, 128, 2), (65, 2048, 3, 0, 1), (90, 512, 2, 32, 4), (33, 4096, 2, 256, 1),
    (70, 1024, 8, 128, 5), (17, 32768, 4, 128, 1), (40, 2048, 4, 128, 11),
    (50, 8192, 2, 0, 2), (21, 16384, 2, 64, 1), (30, 2048, 2, 128, 11),   # 2-bit pair order
]


@pytest.mark.parametrize("d_row,d_col,bits,group,n", CASES)
def test_matvec_against_oracle(d_row, d_col, bits, group, n):
    say("dequant_matvec", d_row, d_col, bits, group, n)
    rng = np.random.default_rng(1000 + d_row + bits)
    words, scales, zeros = packed_layer(rng, d_row, d_col, bits, group)
    check(words, scales, zeros, acts(rng, n, d_col), bits, group, d_col)


def test_matvec_on_gptq_output_and_deterministic():
    # the real packed output of the column solve on a small q_proj-like layer
    torch = _torch()
    say("dequant_matvec on quantize_layer output")
    d_row, d_col, bits, group = 192, 512, 4, 128
    W = synth.gen_weight(101, "mv", d_row, d_col, 0.02, "f16", seed=0)
    X = synth.gen_acts(101, "mvx", 4 * d_col, d_col, "f16", seed=0)
    dev = "cuda:0"
    Wd = torch.from_numpy(W).to(dev)
    H = torch.zeros((d_col, d_col), dtype=torch.float32, device=dev)
    G.hessian_accumulate(H, torch.from_numpy(X).to(dev))
    Gd = G.prepare_hinv(H, damp_frac=0.01, check=True)
    spec = G.Spec.make(bits, group, False, 128, 0.01)
    qw, sc, ze, _ = G.quantize_layer(Wd, Gd, spec)
    xa = X[:3]
    y1 = G.dequant_matvec(qw, sc, ze, torch.from_numpy(xa).to(dev), bits, group, d_col)
    y2 = G.dequant_matvec(qw, sc, ze, torch.from_numpy(xa).to(dev), bits, group, d_col)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    words = qw.cpu().numpy().view(np.uint32)
    check(words, sc.cpu().numpy(), ze.cpu().numpy(), xa, bits, group, d_col)


@pytest.mark.slow
def test_matvec_fullsize_70b_gate():
    # 28672 x 8192 INT4 g128 (the 70B-shaped gate_proj), one activation row, sampled rows
    say("dequant_matvec 28672 x 8192 INT4 g128")
    rng = np.random.default_rng(7)
    d_row, d_col, bits, group = 28672, 8192, 4, 128
    words, scales, zeros = packed_layer(rng, d_row, d_col, bits, group)
    rows = np.sort(rng.choice(d_row, 64, replace=False))
    check(words, scales, zeros, acts(rng, 1, d_col), bits, group, d_col, rows=rows)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_matvec_unaligned_activations(bits):
    """Activation rows two columns past a 16-byte boundary (the 4-byte alignment the entry
    point asks for) with a row stride of d_col + 2: the activations are staged one element at
    a time, in each width's pair order, and the result equals the aligned call's."""
    torch = _torch()
    say("dequant_matvec unaligned x", bits)
    rng = np.random.default_rng(1100 + bits)
    d_row, d_col, group, n = 45, 1024, 128, 3
    words, scales, zeros = packed_layer(rng, d_row, d_col, bits, group)
    x = acts(rng, n, d_col)
    dev = "cuda:0"
    full = torch.zeros((n, d_col + 2), dtype=torch.float16, device=dev)
    full[:, 2:] = torch.from_numpy(x).to(dev)
    xd = full[:, 2:]
    assert xd.stride(0) == d_col + 2 and xd.data_ptr() % 16 != 0 and xd.data_ptr() % 4 == 0
    qw = torch.from_numpy(words.view(np.int32)).to(dev)
    y = G.dequant_matvec(qw, torch.from_numpy(scales).to(dev), torch.from_numpy(zeros).to(dev),
                         xd, bits, group, d_col)
    torch.cuda.synchronize()
    y_al = run_gpu(words, scales, zeros, x, bits, group, d_col)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_al)
    check(words, scales, zeros, x, bits, group, d_col)
