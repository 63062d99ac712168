"""Plain float64 reference of GPTQ layer-wise weight quantization (test infrastructure only).

Sources (cited by page title and section):
  [Q]   page "量化" (Quantization), dingiv.github.io/ai/compute/kernel/quantization
        - section "量化基础" (quantization basics): symmetric form x_q = round(x/s),
          asymmetric form x_q = round(x/s + z), rounding and clipping errors;
        - section "GPTQ": layer objective argmin ||WX - W^X||^2, Hessian H = 2XX^T,
          OBS compensation formula, fixed left-to-right order, Cholesky of H^-1,
          blocks of B = 128 columns with a lazy batch update, per-channel output.
  [G]   page "大模型常见的量化方式" (psvmc.cn), section "按量化粒度划分" (granularity
        table): per-channel and group-wise (128 elements per group) quantization.
  [S]   page "大模型常见的量化方式" (psvmc.cn), section "大模型的分层" (the decoder layer:
        attention q/k/v/o_proj and the MLP gate/up/down_proj, quantized sub-layer by
        sub-layer).
  [L]   page on LLM quantization (m.youleyou.com), section "二、量化是什么" (the
        [-T, T] -> [-127, 127] mapping) and section "四、量化形式" (linear
        quantization with round() and clip() to [qmin, qmax], scale s, offset z).

Readings where the pages are silent or garbled (each function names the one it uses):
  R1  the garbled norm of the objective is the squared Frobenius norm over rows.
  R2  the OBS formula uses the inverse Hessian of the not-yet-quantized set; row q
      of G = Cholesky(H^-1)^T (upper), scaled by G_qq, is that column.
  R3  "Cholesky(H^-1)^T" is the transposed lower Cholesky factor: upper, GᵀG = H^-1.
  R4  natural column order 0..d_col-1, no reordering.
  R5  damping (not on the pages): H_d = H + lambda I, lambda = frac * mean(diag H).
  R6  H is literally 2 X X^T (not averaged).
  R7  group (s, z) are set at the group's first column from the current values.
  R8  symmetric: s = max|x| / (2^(b-1) - 1), signed codes clipped to
      [-2^(b-1), 2^(b-1) - 1], stored with offset z = 2^(b-1).
      asymmetric: range [min(0, min x), max(0, max x)], s = range / (2^b - 1),
      z = round(-xmin / s); degenerate range -> [-1, 1].
  R9  code = clip(round(x/s + z), 0, 2^b - 1), round half to even.
  R13 groups are runs of g consecutive input columns of one row.
  R16 AWQ's exponent grid is n evenly spaced points of [0, 1] with both ends (n = 20);
      s = s_X^alpha is formed in float64 and rounded to float32.
  R17 s_X is the mean |x| of each input channel over all calibration tokens; a channel
      with s_X = 0 keeps s = 1.
  R18 AWQ's loss L(s) is the layer objective ||W X - Q(W diag s) diag(s)^-1 X||^2 with the
      round-to-nearest quantizer of R8/R9 applied to the scaled weights.
  R19 the MLP of a decoder layer (the page lists gate_proj, up_proj and down_proj of the
      LLaMA MLP without its formula) is the LLaMA one: down(silu(gate x) * up x), with
      silu(x) = x sigmoid(x).
  R20 layer-sequential quantization: down_proj is calibrated on the output of the already
      quantized gate_proj and up_proj, rounded to float16 like the block's input.
  R21 the decoder layer (the page lists input_layernorm, self_attn,
      post_attention_layernorm and mlp of the LLaMA layer, norms kept in float16) is the
      LLaMA one: h = x + o_proj(attn(rmsnorm1(x))), and the MLP takes rmsnorm2(h).  Every
      tensor a quantized sub-layer reads (the norm outputs, q/k/v, the attention output O,
      the residual h, the MLP's Y) is stored in float16; the oracle rounds each float64
      value once.
  R22 rmsnorm(x) = x / sqrt(mean(x^2) + eps) * gamma per token, eps = 1e-6.
  R23 attention is LLaMA's causal multi-head self-attention: heads of 128 channels,
      rotary position embedding on q and k (theta = 10000, channel i of a head rotated with
      channel i + 64 by the angle pos * theta^(-2i/128)), positions 0..L-1 within each of
      the independent sequences the calibration tokens are cut into, softmax of
      q k^T / sqrt(128) over the keys at or before the query.
  R15 OBQ's greedy choice is the smallest increase of the row's loss after the OBS
      compensation, (w_p - quant(w_p))^2 / [H_F^-1]_pp, on the per-channel grid of the
      original row; equal increases take the smallest index.
  P1  every decision that turns a float into an integer (z and the codes) is taken
      in float32, the precision of the GPU kernels; the state (current weights,
      H, G, errors) stays float64.

Pins (tests/test_oracle_pins.py): hand-solved 1x2 and 2x3 layers (tests/golden),
brute-force Hessian, G^T G H_d = I and agreement of two independent G routes,
the literal OBS formula with explicit inverses, the conditional least-squares
re-fit, H proportional to I giving round-to-nearest exactly, the identity
sum(e^2) = Delta H_d Delta^T, Delta = E G, blocked = unblocked, invariance to X
scaling, GPTQ <= RTN, grid membership, exact ties, pack/unpack and known words;
dequant_matvec: hand-computed products over known words (INT4, INT3 straddling words,
INT2), the hand-solved 1x2 layer, and sum_t ||W x_t - y_t||^2 = 1/2 sum_r D_r H D_r^T.
obq_greedy_quantize (tests/test_oracle_obq.py): a brute-force greedy by least squares on
the token matrix (order, codes and W^), the literal OBS step in the greedy's own order,
and H proportional to I giving round-to-nearest.
act_absmean, awq_alphas, awq_scales, awq_search (tests/test_oracle_awq.py): a per-token loop
for s_X, the grid's end points, alpha = 0 or flat s_X giving round-to-nearest bit for bit,
every grid loss equal to the output error summed over tokens, the salient-channel effect.
silu, mlp_forward, mlp_block (tests/test_oracle_mlp.py): silu's closed forms, the product
against scalar loops over the code integers, the chain's wiring and its direct-sum losses.
rmsnorm, rope, causal_attention, attn_forward, residual_linear, decoder_block
(tests/test_oracle_block.py): a constant token in closed form and scale invariance, rope on
a unit vector and against its complex form, attention in closed form on head_dim 2, zero
queries giving the running mean, causality, independent sequences, packed identity and
zero weights, the chain's wiring.
No function here is "parity unpinned".
"""

from __future__ import annotations

from typing import Callable, Dict, Optional

import numpy as np

__all__ = [
    "hessian", "damp", "inv_chol_upper", "inv_chol_upper_reversed", "prepare_g",
    "group_params", "quantize_values", "gptq_quantize", "gptq_quantize_obs_literal",
    "rtn_quantize", "dequantize", "layer_loss", "direct_loss", "pack_codes", "unpack_codes",
    "quant_range", "TIE_TOL", "dequant_matvec", "obq_greedy_quantize",
    "act_absmean", "awq_alphas", "awq_scales", "awq_search", "silu", "mlp_forward", "mlp_block",
    "rmsnorm", "rope", "causal_attention", "attn_forward", "residual_linear", "decoder_block",
]

TIE_TOL = 1e-3   # a v within this many steps of k + 1/2 is a near-tie (either code accepted)


# --------------------------------------------------------------------------- a1, a2, a3

def hessian(X, chunk: int = 4096) -> np.ndarray:
    """H = 2 * sum_t x_t x_t^T over the calibration tokens ([Q] GPTQ, Hessian; R6).

    X is token-major [n_tok, d] (row t is the layer input x_t); the sum runs in
    float64 over chunks of tokens.  Each chunk's product x_c^T x_c is one float64 matrix
    product on the host (torch's CPU BLAS, which is several times faster than numpy's at
    the layer sizes of the full-size checks; the definition and the precision are the same).
    """
    import torch
    X = np.asarray(X)
    n, d = X.shape
    acc = torch.zeros((d, d), dtype=torch.float64)
    for t0 in range(0, n, chunk):
        xc = torch.from_numpy(np.ascontiguousarray(X[t0:t0 + chunk])).to(torch.float64)
        acc.addmm_(xc.T, xc)
    return 2.0 * acc.numpy()


def damp(H: np.ndarray, frac: float):
    """H_d = H + lambda*I with lambda = frac * mean(diag H) (R5).  Returns (H_d, lambda)."""
    H = np.asarray(H, dtype=np.float64)
    lam = float(frac) * float(np.mean(np.diag(H)))
    return H + lam * np.eye(H.shape[0]), lam


def inv_chol_upper(Hd: np.ndarray) -> np.ndarray:
    """G = Cholesky(H_d^-1)^T, upper triangular with G^T G = H_d^-1 ([Q] GPTQ, second
    improvement; R3).  Literal route: explicit inverse, then lower Cholesky, then transpose.
    Raises numpy.linalg.LinAlgError when H_d is not positive definite."""
    Hinv = np.linalg.inv(Hd)
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T.copy()


def inv_chol_upper_reversed(Hd: np.ndarray) -> np.ndarray:
    """The same G without forming H_d^-1: factor H_d = U U^T with U upper (a Cholesky of
    the index-reversed matrix, reversed back), then G = U^-1.  Since H_d^-1 = U^-T U^-1,
    G = U^-1 is upper with G^T G = H_d^-1, and the factor with positive diagonal is
    unique, so both routes give the same G.  Float64 LAPACK on the host (torch's CPU
    library: about half the work of the literal route, which matters at d = 28672).
    Raises numpy.linalg.LinAlgError when H_d is not positive definite."""
    import torch
    d = Hd.shape[0]
    A = torch.from_numpy(np.ascontiguousarray(np.asarray(Hd, dtype=np.float64)[::-1, ::-1]))
    L, info = torch.linalg.cholesky_ex(A)
    del A
    if int(info) != 0:
        raise np.linalg.LinAlgError("H_d is not positive definite (pivot %d)" % int(info))
    U = torch.flip(L, dims=(0, 1))
    del L
    G = torch.linalg.solve_triangular(U, torch.eye(d, dtype=torch.float64), upper=True)
    return G.numpy()


def prepare_g(H: np.ndarray, damp_frac: float) -> np.ndarray:
    """Damping (R5) followed by G = Cholesky(H_d^-1)^T."""
    Hd, _ = damp(H, damp_frac)
    return inv_chol_upper(Hd)


# --------------------------------------------------------------------------- quantizer

def quant_range(bits: int):
    """Stored code range [0, 2^b - 1] ([L] 四、量化形式: clip to [qmin, qmax])."""
    return 0, (1 << bits) - 1


def group_params(x: np.ndarray, bits: int, sym: bool):
    """Scale and zero point of each row of a group (R7, R8, P1).

    x: current values [rows, g] (float64 state).  Returns (s float32 [rows],
    z int64 [rows], zf float32 [rows]) where zf is the pre-rounding zero point
    (equal to z for the symmetric form).
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    maxq = (1 << bits) - 1
    one = np.float32(1.0)
    if sym:
        # [L] 二: [-T, T] maps onto the symmetric integer range; [Q] 量化基础: x_q = round(x/s).
        amax = np.max(np.abs(x32), axis=1)
        amax = np.where(amax == 0, one, amax).astype(np.float32)
        s = (amax / np.float32((1 << (bits - 1)) - 1)).astype(np.float32)
        z = np.full(x32.shape[0], 1 << (bits - 1), dtype=np.int64)
        return s, z, z.astype(np.float32)
    # [Q] 量化基础: asymmetric x_q = round(x/s + z) with zero point z.
    xmin = np.minimum(np.min(x32, axis=1), np.float32(0))
    xmax = np.maximum(np.max(x32, axis=1), np.float32(0))
    deg = xmax == xmin
    xmin = np.where(deg, np.float32(-1), xmin).astype(np.float32)
    xmax = np.where(deg, one, xmax).astype(np.float32)
    s = ((xmax - xmin) / np.float32(maxq)).astype(np.float32)
    zf = ((-xmin) / s).astype(np.float32)
    z = np.clip(np.rint(zf), 0, maxq).astype(np.int64)
    return s, z, zf


def quantize_values(w: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int):
    """code = clip(rne(w/s + z), 0, 2^b - 1) decided in float32 (R9, P1).

    Returns (code int64, v float32 pre-rounding value).
    """
    maxq = (1 << bits) - 1
    w32 = np.asarray(w, dtype=np.float64).astype(np.float32)
    v = (w32 / s + z.astype(np.float32)).astype(np.float32)
    code = np.clip(np.rint(v), 0, maxq).astype(np.int64)
    return code, v


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, g: int) -> np.ndarray:
    """W^ = s (code - z) in float64 (exact for float32 s and small integers)."""
    s = np.repeat(np.asarray(scales, dtype=np.float64), g, axis=1)
    z = np.repeat(np.asarray(zeros, dtype=np.float64), g, axis=1)
    return s * (np.asarray(codes, dtype=np.float64) - z)


def _near_tie(v: np.ndarray, tol: float) -> np.ndarray:
    f = v.astype(np.float64) - np.floor(v.astype(np.float64))
    return np.abs(f - 0.5) < tol


# --------------------------------------------------------------------------- a4..a6

TieHook = Callable[[str, int, np.ndarray, np.ndarray, np.ndarray, np.ndarray], np.ndarray]


def gptq_quantize(W, G: np.ndarray, bits: int, group: int, sym: bool,
                  block: Optional[int] = None, tie_hook: Optional[TieHook] = None,
                  tie_tol: float = TIE_TOL) -> Dict[str, np.ndarray]:
    """Column-by-column quantization with OBS compensation, read through G.

    [Q] GPTQ: for q = 0, 1, ... in fixed order (R4): quantize w_q, then move every
    not-yet-quantized weight by delta = -(w_q - quant(w_q)) / [H^-1]_qq * H^-1_{:,q}
    (the inverse over the remaining set, R2).  With G upper and G^T G = H_d^-1 this is
        e = (w_q - w^_q) / G_qq,     w_k -= e * G_qk   for k > q.
    block=None applies every update at once (the definition).  block=B restricts the
    immediate update to the current block of B columns and applies the rest after the
    block as one product W[:, end:] -= E[:, blk] @ G[blk, end:] ([Q] GPTQ, third
    improvement, lazy batch update).

    group: 0 means one group per row (per-output-channel, [Q] GPTQ engineering
    paragraph); g > 0 means runs of g columns ([G]).  (s, z) are set at each group's
    first column from the current values (R7).

    tie_hook(kind, q, rows, own, lo, hi) is consulted only where the float32 value
    that decides an integer lies within tie_tol of k + 1/2 (kind "code" or "zero");
    it returns the value to keep for those rows and must return lo or hi.  It lets a
    caller check another implementation's choice at such ambiguous points; the
    arithmetic here never takes values from it.

    Returns codes [d_row, d_col] (stored, in [0, 2^b-1]), scales float32 and zeros
    [d_row, d_col/g], w_hat float64, E (the e values) float64, V float32 pre-rounding
    values, W_cur the current value of each weight when it was quantized, ties (number
    of positions where the hook changed the choice).
    """
    Wc = np.array(W, dtype=np.float64, copy=True)
    d_row, d_col = Wc.shape
    G = np.asarray(G, dtype=np.float64)
    if G.shape != (d_col, d_col):
        raise ValueError("G must be d_col x d_col")
    g = d_col if group == 0 else int(group)
    if d_col % g:
        raise ValueError("group must divide d_col")
    if block is not None and not (block % g == 0 or g % block == 0):
        raise ValueError("block and group must nest")
    maxq = (1 << bits) - 1

    codes = np.zeros((d_row, d_col), np.int64)
    w_hat = np.zeros((d_row, d_col))
    E = np.zeros((d_row, d_col))
    V = np.zeros((d_row, d_col), np.float32)
    W_cur = np.zeros((d_row, d_col))
    scales = np.zeros((d_row, d_col // g), np.float32)
    zeros = np.zeros((d_row, d_col // g), np.int64)
    ties = 0
    s = z = None
    B = d_col if block is None else int(block)

    for j0 in range(0, d_col, B):
        j1 = min(j0 + B, d_col)
        for q in range(j0, j1):
            if q % g == 0:
                s, z, zf = group_params(Wc[:, q:q + g], bits, sym)
                if tie_hook is not None and not sym:
                    amb = np.nonzero(_near_tie(zf, tie_tol))[0]
                    if amb.size:
                        lo = np.clip(np.floor(zf[amb]), 0, maxq).astype(np.int64)
                        hi = np.clip(lo + 1, 0, maxq)
                        ch = np.asarray(tie_hook("zero", q, amb, z[amb], lo, hi), np.int64)
                        ties += int(np.count_nonzero(ch != z[amb]))
                        z = z.copy()
                        z[amb] = ch
                scales[:, q // g] = s
                zeros[:, q // g] = z
            W_cur[:, q] = Wc[:, q]
            code, v = quantize_values(Wc[:, q], s, z, bits)
            if tie_hook is not None:
                amb = np.nonzero(_near_tie(v, tie_tol))[0]
                if amb.size:
                    lo = np.clip(np.floor(v[amb].astype(np.float64)), 0, maxq).astype(np.int64)
                    hi = np.clip(lo + 1, 0, maxq)
                    keep = lo != hi
                    amb, lo, hi = amb[keep], lo[keep], hi[keep]
                    if amb.size:
                        ch = np.asarray(tie_hook("code", q, amb, code[amb], lo, hi), np.int64)
                        ties += int(np.count_nonzero(ch != code[amb]))
                        code[amb] = ch
            wq = s.astype(np.float64) * (code - z).astype(np.float64)
            e = (Wc[:, q] - wq) / G[q, q]
            codes[:, q] = code
            w_hat[:, q] = wq
            E[:, q] = e
            V[:, q] = v
            Wc[:, q] = wq
            # immediate update of the not-yet-quantized columns inside the block
            Wc[:, q + 1:j1] -= np.outer(e, G[q, q + 1:j1])
        if j1 < d_col:
            # lazy batch update of everything right of the block
            Wc[:, j1:] -= E[:, j0:j1] @ G[j0:j1, j1:]

    return {"codes": codes, "scales": scales, "zeros": zeros, "w_hat": w_hat, "E": E,
            "V": V, "W_cur": W_cur, "ties": ties, "group": g}


def gptq_quantize_obs_literal(W, Hd: np.ndarray, bits: int, group: int, sym: bool):
    """The OBS step of [Q] GPTQ taken literally, for tiny layers only.

    At column q the remaining set is F = {q, ..., d_col-1}; its inverse Hessian
    Hinv_F = inv(H_d[F, F]) is formed explicitly and every remaining weight moves by
    delta_F = -(w_q - quant(w_q)) / [Hinv_F]_qq * [Hinv_F]_{:, q}.  No Cholesky is
    used, so agreement with gptq_quantize checks the reading R2/R3.
    """
    Wc = np.array(W, dtype=np.float64, copy=True)
    d_row, d_col = Wc.shape
    g = d_col if group == 0 else int(group)
    codes = np.zeros((d_row, d_col), np.int64)
    w_hat = np.zeros((d_row, d_col))
    s = z = None
    for q in range(d_col):
        if q % g == 0:
            s, z, _ = group_params(Wc[:, q:q + g], bits, sym)
        code, _ = quantize_values(Wc[:, q], s, z, bits)
        wq = s.astype(np.float64) * (code - z)
        Hinv_F = np.linalg.inv(Hd[q:, q:])
        delta = -np.outer((Wc[:, q] - wq) / Hinv_F[0, 0], Hinv_F[:, 0])
        Wc[:, q:] += delta
        codes[:, q] = code
        w_hat[:, q] = wq
    return {"codes": codes, "w_hat": w_hat, "W_final": Wc}


def obq_greedy_quantize(W, Hd: np.ndarray, bits: int, sym: bool) -> Dict[str, np.ndarray]:
    """Greedy-order quantization (OBQ), the method GPTQ's fixed order replaces ([Q] GPTQ,
    first improvement), one grid per output channel.  Tiny layers only: O(d_row d_col^3).

    Each row is independent.  With F the set of not-yet-quantized columns of a row and
    Hinv_F = inv(H_d[F, F]), quantizing w_p (p in F) and moving the rest of F by the OBS
    compensation raises the row's loss by (w_p - quant(w_p))^2 / [Hinv_F]_pp; the greedy
    step quantizes the p in F with the smallest such increase (R15; equal increases: the
    smallest index), applies that compensation, and drops p from F.  Hinv_F without p
    follows from Hinv_F by eliminating p:  Hinv_F - Hinv_F[:, p] Hinv_F[p, :] / [Hinv_F]_pp
    (the inverse of a principal submatrix).  The grid (s, z) of each row comes from its
    original weights (the per-channel case of R7), so it is the same grid as RTN's and as
    GPTQ's with group 0.  Codes are decided in float32 (R9, P1).

    Returns codes, scales, zeros [d_row, 1], w_hat, and order [d_row, d_col] (the column
    quantized at each step).
    """
    W = np.asarray(W, dtype=np.float64)
    d_row, d_col = W.shape
    Hd = np.asarray(Hd, dtype=np.float64)
    s_all, z_all, _ = group_params(W, bits, sym)
    codes = np.zeros((d_row, d_col), np.int64)
    order = np.zeros((d_row, d_col), np.int64)
    w_hat = np.zeros((d_row, d_col))
    Hinv0 = np.linalg.inv(Hd)
    for r in range(d_row):
        w = W[r].copy()
        s, z = s_all[r:r + 1], z_all[r:r + 1]
        Hinv = Hinv0.copy()
        free = np.ones(d_col, bool)
        for step in range(d_col):
            F = np.nonzero(free)[0]
            code, _ = quantize_values(w[F], np.repeat(s, F.size), np.repeat(z, F.size), bits)
            wq = float(s[0]) * (code - z[0]).astype(np.float64)
            inc = (w[F] - wq) ** 2 / np.diag(Hinv)[F]
            k = int(np.argmin(inc))              # first minimum: the smallest index
            p = int(F[k])
            e = (w[p] - wq[k]) / Hinv[p, p]
            w[F] -= e * Hinv[F, p]
            w[p] = wq[k]
            codes[r, p] = code[k]
            w_hat[r, p] = wq[k]
            order[r, step] = p
            Hinv = Hinv - np.outer(Hinv[:, p], Hinv[p, :]) / Hinv[p, p]
            free[p] = False
    return {"codes": codes, "scales": s_all.reshape(-1, 1), "zeros": z_all.reshape(-1, 1),
            "w_hat": w_hat, "order": order}


def rtn_quantize(W, bits: int, group: int, sym: bool) -> Dict[str, np.ndarray]:
    """Round-to-nearest: the same quantizer on the original weights, no compensation."""
    W = np.asarray(W, dtype=np.float64)
    d_row, d_col = W.shape
    g = d_col if group == 0 else int(group)
    codes = np.zeros((d_row, d_col), np.int64)
    scales = np.zeros((d_row, d_col // g), np.float32)
    zeros = np.zeros((d_row, d_col // g), np.int64)
    for k in range(d_col // g):
        cols = slice(k * g, (k + 1) * g)
        s, z, _ = group_params(W[:, cols], bits, sym)
        scales[:, k] = s
        zeros[:, k] = z
        for c in range(k * g, (k + 1) * g):
            codes[:, c], _ = quantize_values(W[:, c], s, z, bits)
    w_hat = dequantize(codes, scales, zeros, g)
    return {"codes": codes, "scales": scales, "zeros": zeros, "w_hat": w_hat, "group": g}


# --------------------------------------------------------------------------- AWQ search

def act_absmean(X, chunk: int = 4096) -> np.ndarray:
    """s_X: the mean magnitude of each input channel over the calibration tokens ([Q] AWQ;
    R17).  X token-major [n_tok, d]; summed in float64 over chunks of tokens."""
    X = np.asarray(X)
    n, d = X.shape
    acc = np.zeros(d)
    for t0 in range(0, n, chunk):
        acc += np.abs(X[t0:t0 + chunk].astype(np.float64)).sum(axis=0)
    return acc / n


def awq_alphas(n_grid: int = 20) -> np.ndarray:
    """The grid of the exponent: n_grid evenly spaced points of [0, 1], both ends included
    ([Q] AWQ, 20-point grid; R16)."""
    return np.arange(n_grid, dtype=np.float64) / (n_grid - 1)


def awq_scales(sx: np.ndarray, alpha: float) -> np.ndarray:
    """s = s_X^alpha per input channel ([Q] AWQ), formed in float64 and rounded to float32
    (the value every later decision sees; R16).  A channel whose activations are all zero
    keeps s = 1 (R17): it adds nothing to the loss, and 0^alpha would void its weights."""
    sx = np.asarray(sx, dtype=np.float64)
    pw = np.power(np.where(sx > 0, sx, 1.0), float(alpha))
    return np.where(sx > 0, pw, 1.0).astype(np.float32)


def awq_search(W, H: np.ndarray, sx: np.ndarray, bits: int, group: int, sym: bool,
               n_grid: int = 20) -> Dict[str, np.ndarray]:
    """Activation-aware scale search ([Q] AWQ): for each alpha of the grid, scale input
    channel c of W by s_c = s_X[c]^alpha (the activations are divided by the same s, so the
    product is unchanged before quantization), quantize W' = W diag(s) to the nearest grid
    point (rtn_quantize, the quantizer of R8/R9, group parameters from W'), and measure the
    layer objective for the effective weights Q(W') diag(s)^-1 on the calibration inputs:
        L(alpha) = ||W X - Q(W') diag(s)^-1 X||^2 = 1/2 sum_r D_r H D_r^T,
        D = W - Q(W') diag(s)^-1,  H = 2 X X^T undamped (R18).
    alpha* is the first grid point with the smallest loss.  W' is formed in float32 from the
    float32 weights and s (the precision of the GPU path, P1).

    Returns alphas, losses [n_grid], best (index), alpha, s (float32 [d_col]), codes, scales,
    zeros of Q(W') at alpha*, w_hat (the effective weights Q(W') diag(s)^-1) and Wp (W').
    """
    W32 = np.asarray(W, dtype=np.float64).astype(np.float32)
    alphas = awq_alphas(n_grid)
    losses = np.zeros(n_grid)
    keep = None
    for i, a in enumerate(alphas):
        sc = awq_scales(sx, a)
        Wp = (W32 * sc[None, :]).astype(np.float32)
        r = rtn_quantize(Wp, bits, group, sym)
        w_eff = r["w_hat"] / sc.astype(np.float64)[None, :]
        losses[i] = layer_loss(W32, w_eff, H)
        if keep is None or losses[i] < losses[keep[0]]:
            keep = (i, sc, Wp, r, w_eff)
    i, sc, Wp, r, w_eff = keep
    return {"alphas": alphas, "losses": losses, "best": i, "alpha": float(alphas[i]), "s": sc,
            "codes": r["codes"], "scales": r["scales"], "zeros": r["zeros"], "w_hat": w_eff,
            "Wp": Wp, "group": r["group"]}


# --------------------------------------------------------------------------- MLP block

def silu(x):
    """x * sigmoid(x) in float64 (the activation of the LLaMA MLP; R19)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def mlp_forward(X, gate, up, bits: int, group: int, d: int) -> np.ndarray:
    """The MLP's down_proj input from packed gate_proj and up_proj ([S] decoder layer; R19,
    R20): Y = silu(X G^T) * (X U^T) with G, U the dequantized weights, in float64, rounded to
    float16 like the block's own input.  gate and up are (words, scales, zeros) as the column
    solve writes them; X is token-major [n_tok, d]."""
    g = d if group == 0 else int(group)
    Xf = np.asarray(X, dtype=np.float64)
    Gw = dequantize(unpack_codes(gate[0], bits, d), gate[1], gate[2], g)
    Uw = dequantize(unpack_codes(up[0], bits, d), up[1], up[2], g)
    return (silu(Xf @ Gw.T) * (Xf @ Uw.T)).astype(np.float16)


def mlp_block(W_gate, W_up, W_down, X, bits: int, group: int, sym: bool, block: int,
              damp_frac: float) -> Dict[str, object]:
    """Layer-sequential quantization of the MLP of one decoder layer ([S] decoder layer;
    [Q] GPTQ, layer by layer): gate_proj and up_proj on the block input X (one shared H),
    then down_proj on Y = mlp_forward of the quantized gate_proj and up_proj, so the
    quantized sub-layers produce the next sub-layer's calibration input (R20).
    Returns the three gptq_quantize results, Y, and each layer's loss on its own input."""
    H_x = hessian(X)
    G_x = prepare_g(H_x, damp_frac)
    rg = gptq_quantize(W_gate, G_x, bits, group, sym, block)
    ru = gptq_quantize(W_up, G_x, bits, group, sym, block)
    d = np.asarray(X).shape[1]
    gate = (pack_codes(rg["codes"], bits), rg["scales"], rg["zeros"])
    up = (pack_codes(ru["codes"], bits), ru["scales"], ru["zeros"])
    Y = mlp_forward(X, gate, up, bits, group, d)
    H_y = hessian(Y)
    G_y = prepare_g(H_y, damp_frac)
    rd = gptq_quantize(W_down, G_y, bits, group, sym, block)
    return {"gate": rg, "up": ru, "down": rd, "Y": Y, "H_x": H_x, "H_y": H_y,
            "loss_gate": layer_loss(W_gate, rg["w_hat"], H_x),
            "loss_up": layer_loss(W_up, ru["w_hat"], H_x),
            "loss_down": layer_loss(W_down, rd["w_hat"], H_y)}


# --------------------------------------------------------------------------- attention half

def rmsnorm(x, gamma, eps: float = 1e-6) -> np.ndarray:
    """Root-mean-square normalization of each token ([S] decoder layer; R21, R22):
    x / sqrt(mean_c x_c^2 + eps) * gamma in float64, rounded once to float16."""
    xf = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + eps)
    return (xf / r * np.asarray(gamma, dtype=np.float64)[None, :]).astype(np.float16)


def rope(x, pos, theta: float = 10000.0) -> np.ndarray:
    """Rotary position embedding of one head's vectors (R23): x [n, hd] float64, pos [n].
    Channel i (< hd/2) and channel i + hd/2 turn together by pos * theta^(-2i/hd)."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[1]
    half = hd // 2
    inv = theta ** (-(2.0 * np.arange(half)) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=1)


def causal_attention(q, k, v, seq_len: int, head_dim: int = 128) -> np.ndarray:
    """Causal multi-head attention over independent sequences (R23), float64 in and out.
    q, k, v are token-major [n_tok, n_heads * head_dim]; rotary embedding is applied to q
    and k here; the last sequence may be shorter than seq_len."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    n, d = q.shape
    out = np.zeros((n, d))
    for t0 in range(0, n, seq_len):
        t1 = min(n, t0 + seq_len)
        pos = np.arange(t1 - t0)
        mask = pos[None, :] <= pos[:, None]
        for h in range(d // head_dim):
            cs = slice(h * head_dim, (h + 1) * head_dim)
            qh, kh = rope(q[t0:t1, cs], pos), rope(k[t0:t1, cs], pos)
            sc = (qh @ kh.T) / np.sqrt(head_dim)
            sc = np.where(mask, sc, -np.inf)
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out[t0:t1, cs] = p @ v[t0:t1, cs]
    return out


def attn_forward(Xn, qp, kp, vp, bits: int, group: int, seq_len: int,
                 head_dim: int = 128) -> np.ndarray:
    """o_proj's calibration input from the packed q/k/v_proj ([S] decoder layer; R20, R21,
    R23): q, k, v = float16 of X W^T, then causal attention, rounded to float16."""
    d = np.asarray(Xn).shape[1]
    qkv = [dequant_matvec(p[0], p[1], p[2], bits, group, d, Xn).astype(np.float16)
           for p in (qp, kp, vp)]
    return causal_attention(*qkv, seq_len, head_dim).astype(np.float16)


def residual_linear(O, x, op, bits: int, group: int) -> np.ndarray:
    """The residual stream after attention (R21): h = float16(x + O W_o^T)."""
    d = np.asarray(O).shape[1]
    y = dequant_matvec(op[0], op[1], op[2], bits, group, d, O)
    return (np.asarray(x, dtype=np.float64) + y).astype(np.float16)


def decoder_block(W: Dict[str, np.ndarray], x, gamma1, gamma2, seq_len: int, bits: int,
                  group: int, sym: bool, block: int, damp_frac: float,
                  head_dim: int = 128) -> Dict[str, object]:
    """Layer-sequential quantization of one decoder layer ([S] decoder layer; [Q] GPTQ,
    layer by layer; R20, R21): q/k/v_proj on rmsnorm1(x) (one shared H), o_proj on the
    attention output of the quantized q/k/v, gate/up_proj on rmsnorm2(h) with h the residual
    through the quantized o_proj, down_proj on the MLP product of the quantized gate/up.
    W maps the seven sub-layer names to their weights.  Returns each gptq_quantize result,
    every calibration input and Hessian, and each layer's loss on its own input."""
    r: Dict[str, object] = {}

    def run(names, X):
        H = hessian(X)
        G = prepare_g(H, damp_frac)
        out = []
        for nm in names:
            q = gptq_quantize(W[nm], G, bits, group, sym, block)
            r[nm] = q
            r["loss_" + nm] = layer_loss(W[nm], q["w_hat"], H)
            out.append((pack_codes(q["codes"], bits), q["scales"], q["zeros"]))
        return H, out

    n1 = rmsnorm(x, gamma1)
    r["H_n1"], (qp, kp, vp) = run(("q_proj", "k_proj", "v_proj"), n1)
    O = attn_forward(n1, qp, kp, vp, bits, group, seq_len, head_dim)
    r["H_o"], (op,) = run(("o_proj",), O)
    h = residual_linear(O, x, op, bits, group)
    n2 = rmsnorm(h, gamma2)
    r["H_n2"], (gp, up) = run(("gate_proj", "up_proj"), n2)
    Y = mlp_forward(n2, gp, up, bits, group, n2.shape[1])
    r["H_y"], _ = run(("down_proj",), Y)
    r.update(n1=n1, O=O, h=h, n2=n2, Y=Y)
    return r


# --------------------------------------------------------------------------- a8

def layer_loss(W, w_hat, H: np.ndarray) -> float:
    """||W X - W^ X||_F^2 written through H = 2 X X^T: 1/2 * sum_r D_r H D_r^T (R1)."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(w_hat, dtype=np.float64)
    return float(0.5 * np.sum((D @ H) * D))


def direct_loss(W, w_hat, X) -> float:
    """The same objective computed from the activations (X token-major [n_tok, d])."""
    D = np.asarray(W, dtype=np.float64) - np.asarray(w_hat, dtype=np.float64)
    Y = np.asarray(X, dtype=np.float64) @ D.T
    return float(np.sum(Y * Y))


# --------------------------------------------------------------------------- next: W4A16

def dequant_matvec(words: np.ndarray, scales: np.ndarray, zeros: np.ndarray, bits: int,
                   group: int, d_col: int, x) -> np.ndarray:
    """Weight-only quantized linear layer, y = x W^T with W^ read from the packed format:
    y[n, r] = sum_c x[n, c] * s[r, c // g] * (code[r, c] - z[r, c // g]), in float64.

    Page "量化": section GPTQ (the quantized layer computes W X; its output is per-channel
    INT4 for memory-bound single-batch inference) and section AWQ (W4A16: INT4 weights with
    FP16 activations; the dequantization belongs to the matrix product itself, no FP16
    weight matrix is written).  Here the product is taken literally from its definition:
    unpack, dequantize, multiply.  x is [n, d_col] (fp16 values widened), y is [n, d_row].
    """
    g = d_col if group == 0 else group
    codes = unpack_codes(words, bits, d_col)
    w_hat = dequantize(codes, scales, zeros, g)
    return np.asarray(x, dtype=np.float64) @ w_hat.T


# --------------------------------------------------------------------------- a7

def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Code (r, c) occupies bits [c*b, c*b + b) of row r's little-endian bitstream,
    stored as uint32 words [rows, d_col*b/32].  Bit-by-bit, for clarity."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, n = codes.shape
    if (n * bits) % 32:
        raise ValueError("d_col * bits must be a multiple of 32")
    words = np.zeros((rows, n * bits // 32), np.uint64)
    for c in range(n):
        for k in range(bits):
            pos = c * bits + k
            bit = ((codes[:, c] >> k) & 1).astype(np.uint64)
            words[:, pos // 32] |= bit << np.uint64(pos % 32)
    return words.astype(np.uint32)


def unpack_codes(words: np.ndarray, bits: int, n: int) -> np.ndarray:
    words = np.asarray(words, dtype=np.uint64)
    rows = words.shape[0]
    codes = np.zeros((rows, n), np.int64)
    for c in range(n):
        for k in range(bits):
            pos = c * bits + k
            bit = (words[:, pos // 32] >> np.uint64(pos % 32)) & np.uint64(1)
            codes[:, c] |= bit.astype(np.int64) << k
    return codes
