"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each test names what it pins.  None of them re-types the oracle's own formula:
they use hand-solved cases, brute force, explicit inverses, textbook identities,
invariances and exact special cases.
"""

import numpy as np
import pytest

import oracle as O
from tests.golden_io import load_case, load_pack_lines


def _spd(rng, d, n=None):
    n = n or 4 * d
    X = rng.standard_normal((n, d)) * np.exp(0.5 * rng.standard_normal(d))
    return O.hessian(X), X


# ------------------------------------------------------------------ hand-solved layers

def test_hand_1x2():
    c = load_case("hand_1x2.txt")
    H, W = c["H"], c["W"][None, :]
    G = O.prepare_g(H, 0.0)
    np.testing.assert_allclose(G, c["G"], rtol=1e-12, atol=1e-14)
    r = O.gptq_quantize(W, G, bits=3, group=0, sym=False)
    np.testing.assert_array_equal(r["codes"][0], c["codes"])
    np.testing.assert_allclose(r["W_cur"][0, 1], c["w1_compensated"], rtol=1e-6)
    assert r["scales"][0, 0] == c["scale"] and r["zeros"][0, 0] == c["zero"]
    rtn = O.rtn_quantize(W, 3, 0, False)
    np.testing.assert_array_equal(rtn["codes"][0], c["rtn_codes"])
    D = W - r["w_hat"]
    Dr = W - rtn["w_hat"]
    np.testing.assert_allclose((D @ H @ D.T).ravel(), c["quad_loss"], rtol=1e-6)
    np.testing.assert_allclose((Dr @ H @ Dr.T).ravel(), c["rtn_quad_loss"], rtol=1e-6)


def test_hand_2x3():
    c = load_case("hand_2x3.txt")
    H, W = c["H"], c["W"]
    G = O.prepare_g(H, 0.0)
    np.testing.assert_allclose(G, c["G"], rtol=1e-12, atol=1e-14)
    r = O.gptq_quantize(W, G, bits=3, group=0, sym=False)
    np.testing.assert_array_equal(r["codes"], c["codes"])
    np.testing.assert_allclose(r["V"], c["pre_round_v"], rtol=1e-6)
    rtn = O.rtn_quantize(W, 3, 0, False)
    np.testing.assert_array_equal(rtn["codes"], c["rtn_codes"])
    D = W - r["w_hat"]
    np.testing.assert_allclose(np.einsum("ij,jk,ik->i", D, H, D), c["quad_loss"], rtol=1e-6)
    np.testing.assert_allclose(O.layer_loss(W, r["w_hat"], H), c["layer_loss"], rtol=1e-6)
    np.testing.assert_allclose(O.layer_loss(W, rtn["w_hat"], H), c["rtn_layer_loss"], rtol=1e-6)


# ------------------------------------------------------------------ Hessian, damping, G

def test_hessian_brute_force():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((7, 4)).astype(np.float16)
    n, d = X.shape
    ref = [[0.0] * d for _ in range(d)]
    for i in range(d):
        for j in range(d):
            acc = 0.0
            for t in range(n):
                acc += float(X[t, i]) * float(X[t, j])
            ref[i][j] = 2.0 * acc
    H = O.hessian(X, chunk=3)
    np.testing.assert_allclose(H, np.array(ref), rtol=1e-14, atol=1e-14)


def test_hessian_trace_symmetry_psd():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((300, 40))
    H = O.hessian(X, chunk=64)
    assert np.array_equal(H, H.T) or np.allclose(H, H.T, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.trace(H), 2.0 * np.sum(X * X), rtol=1e-12)
    assert np.linalg.eigvalsh(H).min() > 0


def test_damp_value():
    H = np.diag([1.0, 2.0, 6.0]) + 0.5
    Hd, lam = O.damp(H, 0.01)
    assert lam == pytest.approx(0.01 * (1.5 + 2.5 + 6.5) / 3)
    np.testing.assert_allclose(Hd - H, lam * np.eye(3), rtol=1e-12, atol=1e-15)


def test_g_routes_and_inverse():
    rng = np.random.default_rng(3)
    H, _ = _spd(rng, 48)
    Hd, _ = O.damp(H, 0.01)
    G1 = O.inv_chol_upper(Hd)
    G2 = O.inv_chol_upper_reversed(Hd)
    assert np.allclose(np.tril(G1, -1), 0) and np.all(np.diag(G1) > 0)
    np.testing.assert_allclose(G1, G2, rtol=1e-9, atol=1e-12 * np.abs(G1).max())
    np.testing.assert_allclose(G1.T @ G1 @ Hd, np.eye(48), atol=1e-10)


def test_singular_hessian_raises():
    X = np.zeros((10, 4))
    X[:, 0] = 1.0
    H = O.hessian(X)
    with pytest.raises(np.linalg.LinAlgError):
        O.prepare_g(H, 0.0)


# ------------------------------------------------------------------ the column loop

@pytest.mark.parametrize("bits,group,sym", [(4, 0, False), (3, 4, False), (2, 0, False),
                                             (4, 8, True), (3, 0, True)])
def test_literal_obs_formula(bits, group, sym):
    """Compensation through G equals the page's formula with explicit remaining-set inverses."""
    rng = np.random.default_rng(10 + bits + group)
    H, _ = _spd(rng, 16, n=24)
    Hd, _ = O.damp(H, 0.01)
    W = rng.standard_normal((5, 16)) * 0.02
    a = O.gptq_quantize(W, O.inv_chol_upper(Hd), bits, group, sym)
    b = O.gptq_quantize_obs_literal(W, Hd, bits, group, sym)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_allclose(a["w_hat"], b["w_hat"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(b["W_final"], b["w_hat"], rtol=0, atol=1e-12)


def test_conditional_refit():
    """Before column q is quantized its value is the least-squares re-fit of the free
    weights F = {q..} given the already-quantized P = {<q}: w_F + H_FF^-1 H_FP (w_P - w^_P)."""
    rng = np.random.default_rng(11)
    d = 20
    H, _ = _spd(rng, d, n=30)
    Hd, _ = O.damp(H, 0.01)
    W = rng.standard_normal((3, d)) * 0.02
    r = O.gptq_quantize(W, O.inv_chol_upper(Hd), 4, 0, False)
    for q in range(1, d):
        P, F = slice(0, q), slice(q, d)
        refit = W[:, F] + np.linalg.solve(Hd[F, F], Hd[F, P] @ (W[:, P] - r["w_hat"][:, P]).T).T
        np.testing.assert_allclose(r["W_cur"][:, q], refit[:, 0], rtol=1e-9, atol=1e-13)


@pytest.mark.parametrize("bits,group,sym,block", [(4, 0, False, None), (4, 16, True, 32),
                                                   (3, 32, False, 16), (2, 0, False, 64)])
def test_identity_hessian_is_rtn(bits, group, sym, block):
    """H proportional to I makes G diagonal: no compensation, exactly round-to-nearest."""
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((9, 64)) * 0.02).astype(np.float32)
    X = np.eye(64) * 3.0
    G = O.prepare_g(O.hessian(X), 0.01)
    a = O.gptq_quantize(W, G, bits, group, sym, block=block)
    b = O.rtn_quantize(W, bits, group, sym)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["scales"], b["scales"])
    np.testing.assert_array_equal(a["zeros"], b["zeros"])
    np.testing.assert_array_equal(a["w_hat"], b["w_hat"])


def test_error_identities():
    """Delta = W - W^ = E G (row vectors), hence sum_q e_q^2 = Delta H_d Delta^T per row."""
    rng = np.random.default_rng(13)
    H, _ = _spd(rng, 32)
    Hd, _ = O.damp(H, 0.01)
    G = O.inv_chol_upper(Hd)
    W = rng.standard_normal((6, 32)) * 0.02
    r = O.gptq_quantize(W, G, 3, 8, False, block=16)
    D = W - r["w_hat"]
    np.testing.assert_allclose(D, r["E"] @ G, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(np.sum(r["E"] ** 2, axis=1), np.einsum("ij,jk,ik->i", D, Hd, D),
                               rtol=1e-9)


@pytest.mark.parametrize("bits,group,sym", [(4, 128, True), (3, 0, False), (2, 64, False)])
def test_blocked_equals_unblocked(bits, group, sym):
    rng = np.random.default_rng(14)
    d = 512
    H, _ = _spd(rng, d, n=1024)
    G = O.prepare_g(H, 0.01)
    W = rng.standard_normal((8, d)) * 0.02
    ref = O.gptq_quantize(W, G, bits, group, sym)
    for B in (32, 64, 128, 256):
        if not (group == 0 or B % group == 0 or group % B == 0):
            continue
        r = O.gptq_quantize(W, G, bits, group, sym, block=B)
        np.testing.assert_array_equal(r["codes"], ref["codes"])
        np.testing.assert_allclose(r["E"], ref["E"], rtol=1e-9, atol=1e-12)


def test_invariant_to_activation_scale():
    """X -> 2^k X scales H, lambda and G^-2 exactly; codes and scales do not change."""
    rng = np.random.default_rng(15)
    X = rng.standard_normal((200, 48)) * np.exp(0.5 * rng.standard_normal(48))
    W = rng.standard_normal((5, 48)) * 0.02
    a = O.gptq_quantize(W, O.prepare_g(O.hessian(X), 0.01), 4, 16, False)
    b = O.gptq_quantize(W, O.prepare_g(O.hessian(X * 8.0), 0.01), 4, 16, False)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["scales"], b["scales"])


def test_gptq_never_worse_than_rtn_two_columns():
    """With two columns and no damping, column 1 is the grid point nearest the 1-D
    minimiser given the shared column 0, so GPTQ's loss per row is <= RTN's."""
    rng = np.random.default_rng(16)
    worse = 0
    for _ in range(500):
        X = rng.standard_normal((6, 2)) * np.exp(rng.standard_normal(2))
        H = O.hessian(X)
        W = rng.standard_normal((4, 2))
        r = O.gptq_quantize(W, O.prepare_g(H, 0.0), 3, 0, False)
        t = O.rtn_quantize(W, 3, 0, False)
        lg = np.einsum("ij,jk,ik->i", W - r["w_hat"], H, W - r["w_hat"])
        lt = np.einsum("ij,jk,ik->i", W - t["w_hat"], H, W - t["w_hat"])
        worse += int(np.sum(lg > lt * (1 + 1e-9) + 1e-12))
    assert worse == 0


def test_gptq_beats_rtn_on_tiny_layers_in_aggregate():
    """Empirical, on 1000 seeded tiny layers drawn like the 256x256 workload (4x16, 64
    tokens).  Per layer GPTQ is not guaranteed to win (compensation can push a later
    weight outside the row's fixed clip range); in aggregate it must: the summed loss
    is lower, the median ratio is below 1 and most layers improve."""
    ratios, tot_g, tot_r = [], 0.0, 0.0
    for seed in range(1000):
        rng = np.random.default_rng(1000 + seed)
        X = rng.standard_normal((64, 16)) * np.exp(0.5 * rng.standard_normal(16))
        W = rng.standard_normal((4, 16)) * 0.02
        H = O.hessian(X)
        r = O.gptq_quantize(W, O.prepare_g(H, 0.01), 4, 0, False)
        t = O.rtn_quantize(W, 4, 0, False)
        a, b = O.layer_loss(W, r["w_hat"], H), O.layer_loss(W, t["w_hat"], H)
        ratios.append(a / b)
        tot_g += a
        tot_r += b
    ratios = np.array(ratios)
    assert tot_g < 0.95 * tot_r
    assert np.median(ratios) < 0.95
    assert np.mean(ratios < 1) > 0.85


def test_gptq_beats_rtn_on_256_layer():
    """The 256x256 workload shape (1024 tokens, lognormal channel scales, INT4 per row)."""
    rng = np.random.default_rng(19)
    X = rng.standard_normal((1024, 256)) * np.exp(0.5 * rng.standard_normal(256))
    W = rng.standard_normal((256, 256)) * 0.02
    H = O.hessian(X)
    r = O.gptq_quantize(W, O.prepare_g(H, 0.01), 4, 0, False, block=128)
    t = O.rtn_quantize(W, 4, 0, False)
    assert O.layer_loss(W, r["w_hat"], H) < 0.95 * O.layer_loss(W, t["w_hat"], H)


def test_loss_through_h_equals_direct():
    rng = np.random.default_rng(17)
    X = (rng.standard_normal((512, 64)) * np.exp(0.5 * rng.standard_normal(64))).astype(np.float32)
    W = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    H = O.hessian(X)
    r = O.gptq_quantize(W, O.prepare_g(H, 0.01), 4, 0, False, block=32)
    np.testing.assert_allclose(O.layer_loss(W, r["w_hat"], H), O.direct_loss(W, r["w_hat"], X),
                               rtol=1e-9)


# ------------------------------------------------------------------ quantizer

def test_grid_membership_and_ranges():
    rng = np.random.default_rng(18)
    H, _ = _spd(rng, 64)
    W = rng.standard_normal((10, 64)) * 0.02
    for bits, group, sym in [(4, 16, True), (3, 0, False), (2, 32, False), (8, 64, False)]:
        r = O.gptq_quantize(W, O.prepare_g(H, 0.01), bits, group, sym, block=32)
        g = r["group"]
        assert r["codes"].min() >= 0 and r["codes"].max() <= 2 ** bits - 1
        assert r["zeros"].min() >= 0 and r["zeros"].max() <= 2 ** bits - 1
        grid = np.repeat(r["scales"].astype(np.float64), g, 1) * (
            r["codes"] - np.repeat(r["zeros"], g, 1))
        assert np.array_equal(grid, r["w_hat"])
        assert np.array_equal(O.dequantize(r["codes"], r["scales"], r["zeros"], g), r["w_hat"])
        if sym:
            assert np.all(r["zeros"] == 2 ** (bits - 1))


def test_quantizer_known_values():
    # asymmetric 4-bit, group values spanning [-1, 2]: s = 3/15, z = round(1/s) = 5
    s, z, _ = O.group_params(np.array([[-1.0, 0.5, 2.0, 0.25]]), 4, False)
    assert s[0] == np.float32(3.0) / np.float32(15.0) and z[0] == 5
    code, _ = O.quantize_values(np.array([-1.0, 2.0, 0.4, 0.0]), np.repeat(s, 4), np.repeat(z, 4), 4)
    np.testing.assert_array_equal(code, [0, 15, 7, 5])
    # symmetric 4-bit, max |x| = 0.7: s = 0.1, z = 8, -0.7 -> 1, 0.7 -> 15, -0.75 -> 0 (extra code)
    s, z, _ = O.group_params(np.array([[-0.7, 0.3, 0.7]]), 4, True)
    assert s[0] == np.float32(0.7) / np.float32(7.0) and z[0] == 8
    code, _ = O.quantize_values(np.array([-0.7, 0.7, -0.75, 0.0]), np.repeat(s, 4), np.repeat(z, 4), 4)
    np.testing.assert_array_equal(code, [1, 15, 0, 8])
    # all-positive group keeps 0 in range (z = 0), degenerate all-zero group uses [-1, 1]
    s, z, _ = O.group_params(np.array([[1.0, 2.0, 3.0], [0.0, 0.0, 0.0]]), 2, False)
    assert z[0] == 0 and s[0] == np.float32(1.0)
    assert s[1] == np.float32(2.0 / 3.0) and z[1] == 2


def test_exact_ties_round_half_even():
    s = np.full(6, np.float32(1.0))
    z = np.zeros(6, np.int64)
    code, _ = O.quantize_values(np.array([0.5, 1.5, 2.5, 3.5, 14.5, 15.5]), s, z, 4)
    np.testing.assert_array_equal(code, [0, 2, 2, 4, 14, 15])


def test_tie_hook_only_at_near_ties():
    W = np.array([[0.0, 7.0, 2.5004, 3.2]])
    G = np.eye(4)
    seen = []

    def hook(kind, q, rows, own, lo, hi):
        seen.append((kind, q))
        return lo

    r = O.gptq_quantize(W, G, 3, 0, False, tie_hook=hook)
    assert seen == [("code", 2)]
    assert r["codes"][0, 2] == 2 and r["ties"] == 1
    assert O.gptq_quantize(W, G, 3, 0, False)["codes"][0, 2] == 3


# ------------------------------------------------------------------ packing

def test_pack_known_words():
    for bits, codes, words in load_pack_lines():
        got = O.pack_codes(np.array([codes]), bits)
        np.testing.assert_array_equal(got[0], np.array(words, np.uint32))
        np.testing.assert_array_equal(O.unpack_codes(got, bits, len(codes))[0], codes)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_round_trip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 2 ** bits, size=(5, 96))
    np.testing.assert_array_equal(O.unpack_codes(O.pack_codes(codes, bits), bits, 96), codes)
