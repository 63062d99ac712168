"""Pins of the oracle's layer-sequential MLP block (readings R19, R20).

  * silu against closed forms: silu(0) = 0, silu(x) - silu(-x) = x, silu(x) -> x for large x;
  * mlp_forward against scalar Python loops over the code integers (dequantization and the
    two dot products written out element by element), rounded to float16 the same way;
  * mlp_block: Y is the forward pass of the quantized gate_proj and up_proj (and differs
    from the unquantized one), down_proj's loss through H equals the direct token sum, and
    quantizing gate_proj and up_proj on the shared input matches the plain column solve.
"""

import math

import numpy as np

import oracle as O


def test_silu_closed_forms():
    x = np.array([-30.0, -2.5, -1.0, 0.0, 0.5, 3.0, 40.0])
    s = O.silu(x)
    assert s[3] == 0.0
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-12)
    assert abs(s[-1] - 40.0) < 1e-12 and abs(s[0]) < 1e-11
    np.testing.assert_allclose(s[4], 0.5 / (1 + math.exp(-0.5)), rtol=1e-15)


def _packed(rng, rows, d, bits, group):
    g = d if group == 0 else group
    codes = rng.integers(0, 1 << bits, (rows, d))
    scales = rng.uniform(0.01, 0.05, (rows, d // g)).astype(np.float32)
    zeros = rng.integers(0, 1 << bits, (rows, d // g)).astype(np.uint8)
    return codes, scales, zeros


def test_mlp_forward_against_loops():
    rng = np.random.default_rng(5)
    n, d, d_ff, bits, group = 3, 32, 4, 4, 16
    X = (rng.standard_normal((n, d)) * 2).astype(np.float16)
    gc, gs, gz = _packed(rng, d_ff, d, bits, group)
    uc, us, uz = _packed(rng, d_ff, d, bits, group)
    Y = O.mlp_forward(X, (O.pack_codes(gc, bits), gs, gz), (O.pack_codes(uc, bits), us, uz),
                      bits, group, d)
    for t in range(n):
        for j in range(d_ff):
            a = b = 0.0
            for k in range(d):
                x = float(X[t, k])
                a += x * float(gs[j, k // group]) * (int(gc[j, k]) - int(gz[j, k // group]))
                b += x * float(us[j, k // group]) * (int(uc[j, k]) - int(uz[j, k // group]))
            y = np.float16(a / (1.0 + math.exp(-a)) * b)
            # both sides round a float64 value to float16; the sums differ only in order
            assert abs(float(Y[t, j]) - float(y)) <= 2.0 ** -10 * abs(float(y)) + 2.0 ** -24


def test_mlp_block_chain():
    rng = np.random.default_rng(6)
    n, d, d_ff = 512, 64, 128
    X = (rng.standard_normal((n, d)) * np.exp(0.5 * rng.standard_normal(d))).astype(np.float16)
    Wg = rng.standard_normal((d_ff, d)) * 0.05
    Wu = rng.standard_normal((d_ff, d)) * 0.05
    Wd = rng.standard_normal((d, d_ff)) * 0.05
    r = O.mlp_block(Wg, Wu, Wd, X, 4, 32, False, 32, 0.01)
    gate = (O.pack_codes(r["gate"]["codes"], 4), r["gate"]["scales"], r["gate"]["zeros"])
    up = (O.pack_codes(r["up"]["codes"], 4), r["up"]["scales"], r["up"]["zeros"])
    np.testing.assert_array_equal(r["Y"], O.mlp_forward(X, gate, up, 4, 32, d))
    Xf = X.astype(np.float64)
    Y_full = (O.silu(Xf @ Wg.T) * (Xf @ Wu.T)).astype(np.float16)
    assert not np.array_equal(r["Y"], Y_full)
    np.testing.assert_allclose(r["loss_down"], O.direct_loss(Wd, r["down"]["w_hat"], r["Y"]),
                               rtol=1e-9)
    G_x = O.prepare_g(O.hessian(X), 0.01)
    np.testing.assert_array_equal(r["gate"]["codes"],
                                  O.gptq_quantize(Wg, G_x, 4, 32, False, 32)["codes"])
    assert r["loss_down"] > 0 and r["loss_gate"] > 0
