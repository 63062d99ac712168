"""Pins of the oracle's attention half of the decoder layer (readings R21-R23).

  * rmsnorm: a constant token against its closed form, invariance to scaling a token,
    and the per-token sum of squares written as a scalar loop;
  * rope: position 0 is the identity, a unit vector on channel 0 turns into
    (cos p, sin p) on channels 0 and hd/2 (the pairing and the direction), pair norms are
    kept, and the same rotation written with complex numbers;
  * causal_attention: closed forms on head_dim 2 (scores cos(m - n)/sqrt2 and
    sin(m - n)/sqrt2 from fixed q and k), q = 0 giving the running mean of v, the first
    token of every sequence returning its own v, causality and independent sequences;
  * attn_forward / residual_linear: packed identity and zero weights reduce them to the
    running mean of the input and to x + O;
  * decoder_block: every calibration input is the forward pass of the quantized
    sub-layers before it, and differs from the unquantized one; the losses equal the
    direct sums over tokens.
"""

import math

import numpy as np

import oracle as O


def test_rmsnorm_closed_forms():
    gamma = np.array([1.0, 2.0, 0.5, 1.5], np.float16)
    for c in (3.0, -0.25):
        y = O.rmsnorm(np.full((1, 4), c), gamma)
        want = np.sign(c) * gamma.astype(np.float64) / math.sqrt(1.0 + 1e-6 / (c * c))
        np.testing.assert_array_equal(y[0], want.astype(np.float16))
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64)) * 3
    g = np.exp(0.2 * rng.standard_normal(64)).astype(np.float16)
    y = O.rmsnorm(x, g)
    for t in range(5):
        ss = 0.0
        for c in range(64):
            ss += x[t, c] * x[t, c]
        r = math.sqrt(ss / 64 + 1e-6)
        for c in range(64):
            v = np.float16(x[t, c] / r * float(g[c]))
            assert abs(float(y[t, c]) - float(v)) <= 2.0 ** -11 * abs(float(v))
    # the norm of a token does not depend on its scale (eps aside)
    y2 = O.rmsnorm(x * 1000.0, g)
    assert np.max(np.abs(y2.astype(np.float64) - y.astype(np.float64)) /
                  np.abs(y.astype(np.float64))) <= 2.0 ** -10


def test_rope_pins():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 128))
    np.testing.assert_array_equal(O.rope(x[:1], [0]), x[:1])
    e0 = np.zeros((3, 128))
    e0[:, 0] = 1.0
    pos = np.array([1.0, 5.0, 2047.0])
    r = O.rope(e0, pos)
    np.testing.assert_allclose(r[:, 0], np.cos(pos), rtol=0, atol=1e-15)
    np.testing.assert_allclose(r[:, 64], np.sin(pos), rtol=0, atol=1e-15)
    assert np.count_nonzero(np.delete(r, [0, 64], axis=1)) == 0
    p = np.arange(6) * 37.0
    y = O.rope(x, p)
    np.testing.assert_allclose(np.hypot(y[:, :64], y[:, 64:]), np.hypot(x[:, :64], x[:, 64:]),
                               rtol=1e-13)
    # complex form: z_i = x_i + j x_{i+64} times exp(j p 10000^(-i/64))
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * p[:, None] * 10000.0 ** (-np.arange(64) / 64))
    np.testing.assert_allclose(y, np.concatenate([z.real, z.imag], axis=1), rtol=0, atol=1e-12)


def test_attention_closed_forms_head_dim_2():
    L = 7
    v = np.random.default_rng(3).standard_normal((L, 2))
    m = np.arange(L)
    for k0, f in (((1.0, 0.0), np.cos), ((0.0, 1.0), np.sin)):
        q = np.tile([1.0, 0.0], (L, 1))
        k = np.tile(k0, (L, 1))
        out = O.causal_attention(q, k, v, L, head_dim=2)
        for i in range(L):
            w = np.exp(f(m[i] - m[: i + 1]) / math.sqrt(2.0))
            np.testing.assert_allclose(out[i], w @ v[: i + 1] / w.sum(), rtol=1e-13)


def test_attention_structure():
    rng = np.random.default_rng(4)
    n, d, L = 300, 256, 128
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    out = O.causal_attention(q, k, v, L)
    starts = np.arange(0, n, L)
    np.testing.assert_allclose(out[starts], v[starts], rtol=1e-14)
    # q = 0: every key weighs the same, so the output is the running mean of v
    z = O.causal_attention(np.zeros_like(q), k, v, L)
    for t0 in starts:
        seg = v[t0:t0 + L]
        np.testing.assert_allclose(z[t0:t0 + L], np.cumsum(seg, 0) / np.arange(1, len(seg) + 1)[:, None],
                                   rtol=1e-12, atol=1e-14)
    # causality: later tokens do not change earlier outputs
    k2, v2 = k.copy(), v.copy()
    k2[200:], v2[200:] = 0.0, 5.0
    np.testing.assert_array_equal(O.causal_attention(q, k2, v2, L)[:200], out[:200])
    # sequences are independent and each restarts at position 0
    np.testing.assert_allclose(O.causal_attention(q[128:256], k[128:256], v[128:256], L),
                               out[128:256], rtol=1e-13)


def _identity_pack(d, bits=4):
    codes = np.eye(d, dtype=np.int64)
    return O.pack_codes(codes, bits), np.ones((d, 1), np.float32), np.zeros((d, 1), np.uint8)


def _zero_pack(d, bits=4):
    codes = np.full((d, d), 3, np.int64)
    return O.pack_codes(codes, bits), np.ones((d, 1), np.float32), np.full((d, 1), 3, np.uint8)


def test_attn_forward_and_residual_reduce():
    rng = np.random.default_rng(5)
    n, d, L = 200, 128, 64
    X = rng.standard_normal((n, d)).astype(np.float16)
    Ob = O.attn_forward(X, _zero_pack(d), _zero_pack(d), _identity_pack(d), 4, 0, L)
    Xf = X.astype(np.float64)
    for t0 in range(0, n, L):
        seg = Xf[t0:t0 + L]
        want = np.cumsum(seg, 0) / np.arange(1, len(seg) + 1)[:, None]
        # one rounding of a float64 value whose summation order differs: within one step
        step = np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(Ob[t0:t0 + L].astype(np.float64) - want) <= step)
    x = rng.standard_normal((n, d)).astype(np.float16)
    h = O.residual_linear(Ob, x, _identity_pack(d), 4, 0)
    np.testing.assert_array_equal(h, (x.astype(np.float64) + Ob.astype(np.float64)).astype(np.float16))


def test_decoder_block_chain():
    rng = np.random.default_rng(6)
    n, d, d_ff, L = 300, 128, 192, 128
    x = (rng.standard_normal((n, d)) * np.exp(0.5 * rng.standard_normal(d))).astype(np.float16)
    g1 = np.exp(0.2 * rng.standard_normal(d)).astype(np.float16)
    g2 = np.exp(0.2 * rng.standard_normal(d)).astype(np.float16)
    shapes = {"q_proj": (d, d), "k_proj": (d, d), "v_proj": (d, d), "o_proj": (d, d),
              "gate_proj": (d_ff, d), "up_proj": (d_ff, d), "down_proj": (d, d_ff)}
    W = {k: rng.standard_normal(s) * 0.08 for k, s in shapes.items()}
    bits, group = 4, 32
    r = O.decoder_block(W, x, g1, g2, L, bits, group, False, 32, 0.01)
    pk = {k: (O.pack_codes(r[k]["codes"], bits), r[k]["scales"], r[k]["zeros"]) for k in shapes}
    np.testing.assert_array_equal(r["n1"], O.rmsnorm(x, g1))
    Oq = O.attn_forward(r["n1"], pk["q_proj"], pk["k_proj"], pk["v_proj"], bits, group, L)
    np.testing.assert_array_equal(r["O"], Oq)
    xf = r["n1"].astype(np.float64)
    O_full = O.causal_attention(*(xf @ W[k].T for k in ("q_proj", "k_proj", "v_proj")), L)
    assert not np.array_equal(r["O"], O_full.astype(np.float16))
    np.testing.assert_array_equal(r["h"], O.residual_linear(r["O"], x, pk["o_proj"], bits, group))
    np.testing.assert_array_equal(r["n2"], O.rmsnorm(r["h"], g2))
    np.testing.assert_array_equal(r["Y"], O.mlp_forward(r["n2"], pk["gate_proj"], pk["up_proj"],
                                                        bits, group, d))
    for k, X in (("q_proj", r["n1"]), ("v_proj", r["n1"]), ("o_proj", r["O"]),
                 ("up_proj", r["n2"]), ("down_proj", r["Y"])):
        np.testing.assert_allclose(r["loss_" + k], O.direct_loss(W[k], r[k]["w_hat"], X), rtol=1e-9)
    G1 = O.prepare_g(O.hessian(r["n1"]), 0.01)
    np.testing.assert_array_equal(r["k_proj"]["codes"],
                                  O.gptq_quantize(W["k_proj"], G1, bits, group, False, 32)["codes"])
