"""The blocked inverse-factor schedule (gptq_prepare_plan), checked on the host:

  * executed launch by launch in float64 NumPy, every buffer entry the schedule must not
    read (the lower triangle of the matrix, the U and tree scratch) starting as NaN, it
    gives the oracle's G = Cholesky(H_d^-1)^T (page "量化", GPTQ, Cholesky
    reformulation) to rounding, with U = G^-1 (U U^T = H_d) above the diagonal blocks of
    the U scratch;
  * the parts of one launch (the leaf's workgroup and the products' tiles run at the same
    time) never touch the same entries with one of them writing (accesses as rectangles,
    so the check is conservative); launches run in stream order;
  * the launch count and the placement of the work: one leaf per 128-block, every tree
    product exactly once, each after the launches that complete its inputs;
  * with the enclosing node's Q = P G22 carried along (the block as the left half of a
    recursion node), Q comes out equal to P times the upper triangle of G22, its K chunks
    in consecutive launches, and the rest as without it.
"""

import numpy as np
import pytest

import oracle as O
from post_weight_quantization_24_amd import gptq as G

FUSED, GEMM = 0, 1


def _gemm(rec):
    names = ("M", "N", "K", "Ab", "Ao", "Al", "tA", "triA", "Bb", "Bo", "Bl", "tB", "triB",
             "Cb", "Co", "Cl", "triC", "alpha", "beta", "t0", "t1")
    return dict(zip(names, (int(v) for v in rec)))


def _ops(n, r=0):
    head, ops = G.prepare_plan(n, r=r)
    out = []
    for r in ops:
        o = dict(kind=int(r[0]), off=int(r[3]), n=int(r[4]))
        o["g"] = [_gemm(r[5 + 21 * j:26 + 21 * j]) for j in range(int(r[1]))]
        out.append(o)
    return head, out


def _tiles(g):
    """Row and column ranges of the tiles [t0, t1) of one product, in the GEMM's tile order
    (by rows; by columns for a lower op(B), by columns from the last for an upper op(B); by
    rows from the last for a lower op(A))."""
    e = 64
    tm, tn = -(-g["M"] // e), -(-g["N"] // e)
    order = 1 if g["triB"] == 2 else 2 if g["triB"] == 1 else 3 if g["triA"] == 2 else 0
    out = []
    for t in range(g["t0"], g["t1"]):
        if order in (1, 2):
            i, j = t % tm, t // tm
            if order == 2:
                j = tn - 1 - j
        else:
            i, j = t // tn, t % tn
            if order == 3:
                i = tm - 1 - i
        out.append((i * e, min(i * e + e, g["M"]), j * e, min(j * e + e, g["N"])))
    return out


def _view(bufs, b, off, rows, cols, ld):
    flat = bufs[b].reshape(-1)
    assert off + (rows - 1) * ld + cols <= flat.size
    return np.lib.stride_tricks.as_strided(flat[off:], shape=(rows, cols),
                                           strides=(ld * 8, 8), writeable=True)


def _run_gemm(bufs, g):
    M, N, K = g["M"], g["N"], g["K"]
    A = _view(bufs, g["Ab"], g["Ao"], *((K, M) if g["tA"] else (M, K)), g["Al"])
    B = _view(bufs, g["Bb"], g["Bo"], *((N, K) if g["tB"] else (K, N)), g["Bl"])
    opA = (A.T if g["tA"] else A).copy()
    opB = (B.T if g["tB"] else B).copy()
    if g["triA"] == 1:
        opA[np.tril_indices(M, -1, K)] = 0.0
    elif g["triA"] == 2:
        opA[np.triu_indices(M, 1, K)] = 0.0
    if g["triB"] == 1:
        opB[np.tril_indices(K, -1, N)] = 0.0
    elif g["triB"] == 2:
        opB[np.triu_indices(K, 1, N)] = 0.0
    C = _view(bufs, g["Cb"], g["Co"], M, N, g["Cl"])
    for r0, r1, c0, c1 in _tiles(g):
        new = g["alpha"] * (opA[r0:r1] @ opB[:, c0:c1])
        if g["beta"]:
            new = new + C[r0:r1, c0:c1]
        if g["triC"]:
            keep = np.arange(r0, r1)[:, None] <= np.arange(c0, c1)[None, :]
            C[r0:r1, c0:c1] = np.where(keep, new, C[r0:r1, c0:c1])
        else:
            C[r0:r1, c0:c1] = new


def _execute(A_upper, n, r=0, G22=None, P=None):
    """Runs the schedule of the n-block in an (n + r)-square matrix; with r > 0, G22 (upper,
    r x r) sits right below and right of the block and P (n x r) is buffer 3."""
    head, ops = _ops(n, r)
    panel, qs = int(head[2]), int(head[3])
    ld = n + r
    mat = np.full((ld, ld), np.nan)
    iu = np.triu_indices(n)
    mat[:n, :n][iu] = A_upper[iu]
    if r:
        mat[n:, n:][np.triu_indices(r)] = G22[np.triu_indices(r)]
    bufs = [mat, np.full(panel, np.nan), np.full(max(qs, 1), np.nan),
            P.copy() if r else np.full(1, np.nan), np.full((max(n * r, 1),), np.nan)]
    for o in ops:
        if o["n"] > 0:
            a, m = o["off"], o["n"]
            blk = mat[a:a + m, a:a + m]
            S = np.triu(blk) + np.triu(blk, 1).T
            Gk = O.inv_chol_upper(S)
            bi = np.triu_indices(m)
            blk[bi] = Gk[bi]
        for g in o["g"]:
            _run_gemm(bufs, g)
    return mat[:n, :n], bufs[1].reshape(n, n), bufs[4].reshape(n, r) if r else None


def _spd(n, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n + 64, n))
    X[:, 3] *= 30.0                        # an outlier channel, as in the outlier workload
    H = 2.0 * X.T @ X
    Hd, _ = O.damp(H, 0.01)
    return Hd


@pytest.mark.parametrize("n", [256, 1100, 2048])
def test_schedule_computes_the_factor(n):
    Hd = _spd(n, 7 + n)
    got, Us, _ = _execute(Hd, n)
    ref = O.inv_chol_upper(Hd)
    up = np.triu(got)
    assert np.all(np.isfinite(up))
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.max(np.abs(up - ref) / scale) < 1e-9
    # the U scratch above the diagonal blocks: U = G^-1, U U^T = H_d
    U = np.linalg.inv(ref)
    assert np.max(np.abs(U @ U.T - Hd)) < 1e-9 * np.abs(Hd).max()
    nb = (n + 127) // 128
    for k in range(1, nb):
        c0, c1 = 128 * k, min(128 * k + 128, n)
        assert np.max(np.abs(Us[:c0, c0:c1] - U[:c0, c0:c1])) < 1e-9 * np.abs(U).max()


def _parts(o, n, ld=None, r=0):
    """Accesses of each part of one launch: [(buffer, row0, row1, col0, col1, writes)] for
    the leaf and for each product (its operands whole, its output tile by tile); buffer 2
    (the tree scratch) is addressed as one column."""
    parts = []
    ld0 = n if ld is None else ld

    def rect(acc, b, off, rows, cols, ld, w, r_in=None):
        if b == 1:
            assert ld == n
        if b == 0:
            assert ld == ld0
        if b in (3, 4):
            assert ld == r
        if b == 2:
            lo = off + (r_in[0] * ld if r_in else 0)
            hi = off + ((r_in[1] - 1) * ld + cols if r_in else (rows - 1) * ld + cols)
            acc.append((b, lo, hi, 0, 1, w))
        else:
            r0, c0 = divmod(off, ld)
            acc.append((b, r0, r0 + rows, c0, c0 + cols, w))

    if o["n"] > 0:
        acc = []
        rect(acc, 0, o["off"] * ld0 + o["off"], o["n"], o["n"], ld0, True)
        parts.append(acc)
    for g in o["g"]:
        acc = []
        M, N, K = g["M"], g["N"], g["K"]
        rect(acc, g["Ab"], g["Ao"], *((K, M) if g["tA"] else (M, K)), g["Al"], False)
        rect(acc, g["Bb"], g["Bo"], *((N, K) if g["tB"] else (K, N)), g["Bl"], False)
        for r0, r1, c0, c1 in _tiles(g):
            if g["Cb"] == 2:
                rect(acc, 2, g["Co"] + c0, r1 - r0, c1 - c0, g["Cl"], True, (r0, r1))
            else:
                rect(acc, g["Cb"], g["Co"] + r0 * g["Cl"] + c0, r1 - r0, c1 - c0, g["Cl"], True)
        parts.append(acc)
    return parts


def _overlap(a, b):
    return a[0] == b[0] and a[1] < b[2] and b[1] < a[2] and a[3] < b[4] and b[3] < a[4]


@pytest.mark.parametrize("n,r", [(1024, 0), (1100, 0), (2048, 0), (4096, 0), (1024, 1024),
                                 (1536, 1600), (2048, 2048)])
def test_launch_parts_are_disjoint(n, r):
    head, ops = _ops(n, r)
    conflicts = 0
    for o in ops:
        parts = _parts(o, n, n + r, r)
        for i in range(len(parts)):
            for j in range(i + 1, len(parts)):
                for a in parts[i]:
                    for b in parts[j]:
                        if (a[5] or b[5]) and _overlap(a, b):
                            conflicts += 1
    assert conflicts == 0


@pytest.mark.parametrize("n", [1024, 1100, 4096])
def test_launch_structure(n):
    head, ops = _ops(n)
    nb = (n + 127) // 128
    assert int(head[0]) == nb and int(head[4]) == len(ops)
    leaves = [o["off"] for o in ops if o["n"] > 0]
    assert leaves == [128 * k for k in range(nb - 1, -1, -1)]      # bottom right first
    assert all(o["kind"] == FUSED for o in ops if o["n"] > 0)
    assert all(len(o["g"]) <= 6 for o in ops)
    # the chain: 3 launches per block but the last (leaf, panel, column), then the tree's
    # remaining levels.  The tree's products (a buffer-2 operand) are 2 per node, nb - 1
    # nodes, and their tile ranges cover each product exactly once, in order.
    assert len(ops) >= 3 * nb - 2
    cover = {}
    for o in ops:
        for g in o["g"]:
            if g["Cb"] == 2 or g["Bb"] == 2:
                key = (g["Cb"], g["Co"], g["Bb"], g["Bo"])
                assert cover.get(key, 0) == g["t0"]
                cover[key] = g["t1"]
            else:
                assert g["t0"] == 0
            assert g["t1"] <= -(-g["M"] // 64) * -(-g["N"] // 64)
    assert len(cover) == 2 * (nb - 1)
    for (cb, co, bb, bo), t1 in cover.items():
        g = next(g for o in ops for g in o["g"] if (g["Cb"], g["Co"], g["Bb"], g["Bo"]) == (cb, co, bb, bo))
        assert t1 == -(-g["M"] // 64) * -(-g["N"] // 64)


@pytest.mark.parametrize("n,r", [(1024, 1024), (1100, 900)])
def test_schedule_carries_the_node_q(n, r):
    rng = np.random.default_rng(n + r)
    Hd = _spd(n, 11 + n)
    G22 = np.triu(rng.standard_normal((r, r))) + 4.0 * np.eye(r)
    P = rng.standard_normal((n, r))
    got, _, Q = _execute(Hd, n, r, G22, P)
    ref = O.inv_chol_upper(Hd)
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.max(np.abs(np.triu(got) - ref) / scale) < 1e-9
    Qr = P @ np.triu(G22)
    assert np.max(np.abs(Q - Qr)) < 1e-9 * np.abs(Qr).max()
    # the chunks: consecutive K ranges of at most 512, each in a later launch
    head, ops = _ops(n, r)
    assert int(head[1]) == r
    where = [(i, g) for i, o in enumerate(ops) for g in o["g"] if g["Cb"] == 4]
    k0s = sorted({g["Bo"] // (n + r) - n for _, g in where})
    assert k0s == list(range(0, r, 512))
    last = {}
    for i, g in where:
        k0 = g["Bo"] // (n + r) - n
        assert g["beta"] == (0 if k0 == 0 else 1) and g["K"] == min(512, r - k0)
        last[k0] = max(last.get(k0, -1), i)
        if k0 > 0:
            assert i > last[k0 - 512]


def test_plan_rejects_bad_sizes():
    lib = G.lib()
    assert lib.gptq_prepare_plan(0, 10, 0, None, 0) == G.EINVAL
    assert lib.gptq_prepare_plan(100, 99, 0, None, 0) == G.EINVAL
    assert lib.gptq_prepare_plan(100, 150, 60, None, 0) == G.EINVAL   # ld < n + r
    assert lib.gptq_prepare_plan(100, 100, -1, None, 0) == G.EINVAL
    assert lib.gptq_prepare_plan(128, 128, 0, None, 0) == 2   # header and the single leaf
