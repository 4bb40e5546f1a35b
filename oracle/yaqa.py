"""fp64 reference of rounding with output-side feedback (generalized LDLQ of
YAQA) on KronQ's Kronecker sketch. TEST INFRASTRUCTURE ONLY (see the package
header): nothing on the product path imports it.

Source (cited by page and section only):
  [YQ]  Notes on YAQA (arXiv 2505.22988), section "关键设计" (key designs):
        item 1 (structural nilpotency: for a Kronecker factor L = L_O (x) L_I
        the fixed-point iteration of the rounding settles within
        snd(L_O) + snd(L_I) <= m + n - 1 steps) and item 4 (the generalized
        LDLQ update, Eq. 5/6: W = Q(W* + L_O'^T Delta L_I' + L_O'^T Delta +
        Delta L_I') with Delta = W* - W and L' = L - I); section "损失函数 /
        训练策略" (the proxy objective tr(Delta^T H_O Delta H_I) that the
        rounding minimises for the sketch H ~ H_O (x) H_I).

Notation: W is d_out x d_in (m x n), rows are output channels. H_I (n x n)
is the input-side factor and H_O (m x m) the output-side factor.

Readings:
  R-Y1  The triangular factors are those of H = A D A^T with A unit UPPER
        triangular, for rows and columns visited in increasing index (QuIP's
        LDLQ convention, under which LDLQ equals GPTQ). With that factor the
        rounding residuals decouple: tr(Delta H_I Delta^T H_O) =
        sum_ij eps_ij^2 D_O,i D_I,j (pinned in the tests). The pages' L' is
        A - I, the strictly upper part.
  R-Y2  The sketch is KronQ's own: H_I = H_X' and H_O = H_G' after BiIP,
        each damped by 1% of its mean diagonal, as the KronQ path damps H_X.
  R-Y3  The target W* is W0 (no drift), or the GPTAQ fold W0 + W0 P when the
        drift term is used: the same matrix the KronQ sweep rounds.
  R-Y4  One grid per output channel, from W0 (before the fold), as the KronQ
        sweep takes it. Group grids depend on the moment a row reaches a
        group, which the two-sided order does not fix; they are out of scope.
"""
from __future__ import annotations

import numpy as np

from .kronq import _quantize, grid_fp32


def ldl_upper(H):
    """(A, d) with H = A diag(d) A^T, A unit upper triangular, d > 0.

    Definition written out: the Cholesky factor of the index-reversed matrix,
    J H J = L L^T, gives H = (J L J)(J L J)^T with J L J upper triangular;
    A scales its columns to a unit diagonal and d holds the squared diagonal.
    Raises LinAlgError if H is not positive definite.
    """
    H = np.asarray(H, dtype=np.float64)
    L = np.linalg.cholesky(H[::-1, ::-1])
    R = L[::-1, ::-1]
    r = np.diag(R).copy()
    return R / r[None, :], r * r


def _grid_arrays(scale, zero, m):
    sc = np.broadcast_to(np.asarray(scale, dtype=np.float32).reshape(-1), (m,)).copy()
    zr = np.broadcast_to(np.asarray(zero, dtype=np.float32).reshape(-1), (m,)).copy()
    return sc, zr


def fixed_point(Wt, H_in, H_out, scale, zero, bits: int, iters: int | None = None):
    """The rounding as the pages state it: the fixed-point iteration of
    [YQ] key design 4, Eq. 5/6,
        W <- Q(W* + L_O'^T Delta L_I' + L_O'^T Delta + Delta L_I'),
        Delta = W* - W,
    started from W = Q(W*), with L' = A - I from ldl_upper of the (already
    damped) factors H_in (n x n) and H_out (m x m). Q rounds each entry on its
    row's grid. Runs ``iters`` iterations (default m + n - 1, the bound of
    [YQ] key design 1) and returns (codes, what, changed) where ``changed`` is
    True if one more iteration would still change a code.
    """
    Wt = np.asarray(Wt, dtype=np.float64)
    m, n = Wt.shape
    sc, zr = _grid_arrays(scale, zero, m)
    maxq = 2 ** bits - 1
    Li = ldl_upper(H_in)[0] - np.eye(n)
    Lo = ldl_upper(H_out)[0] - np.eye(m)
    sc64 = sc.astype(np.float64)[:, None]
    zr64 = zr.astype(np.float64)[:, None]

    def rnd(Z):
        q, _ = _quantize(Z, sc[:, None], zr[:, None], maxq)
        return q, sc64 * (q - zr64)

    q, W = rnd(Wt)
    for _ in range(m + n - 1 if iters is None else iters):
        Dl = Wt - W
        q, W = rnd(Wt + Lo.T @ Dl @ Li + Lo.T @ Dl + Dl @ Li)
    Dl = Wt - W
    q2, _ = rnd(Wt + Lo.T @ Dl @ Li + Lo.T @ Dl + Dl @ Li)
    return q.astype(np.uint8), W, bool(np.any(q2 != q))


def round_two_sided(Wt, U_in, U_out, scale, zero, bits: int, forced_codes=None):
    """The same rounding, element by element in row-major order.

    Row-major order is one of the orders the fixed point allows (an entry
    depends only on entries above-left of it). In terms of the inverse
    factors (U^T U = H^-1, U = D^-1/2 A^-1) the feedback of Eq. 5/6 becomes
        z_ij = W*_ij - sum_{k <= i, l <= j, (k,l) != (i,j)} U_out[k,i] e_kl U_in[l,j],
        e_kl = (z_kl - w^_kl) / (U_out[k,k] U_in[l,l]),
    which with U_out = I is the GPTQ column update of the KronQ sweep. That
    this equals fixed_point() is pinned in the tests, not assumed.

    Per row i: the rows above enter through M_k = e_k U_in (complete rows,
    U_in upper keeps l <= j), the row itself through its running sum
    t_j = sum_{l<j} e_il U_in[l,j].

    Forced replay: with ``forced_codes``, each code that differs from the
    oracle's is recorded as (row, col, oracle code, forced code, distance of
    the oracle's pre-rounding value to the midpoint of the two codes in grid
    steps), and the forced code is adopted.

    Returns dict(codes, what, eps (z - w^), mismatches).
    """
    Wt = np.asarray(Wt, dtype=np.float64)
    U_in = np.asarray(U_in, dtype=np.float64)
    U_out = np.asarray(U_out, dtype=np.float64)
    m, n = Wt.shape
    sc, zr = _grid_arrays(scale, zero, m)
    maxq = 2 ** bits - 1
    codes = np.zeros((m, n), dtype=np.uint8)
    what = np.zeros((m, n))
    eps = np.zeros((m, n))
    M = np.zeros((m, n))
    mism = []
    for i in range(m):
        base = Wt[i] - U_out[:i, i] @ M[:i]
        t = np.zeros(n)
        e = np.zeros(n)
        uo = U_out[i, i]
        s32, z32 = sc[i:i + 1], zr[i:i + 1]
        s64, z64 = float(sc[i]), float(zr[i])
        for j in range(n):
            z = base[j] - uo * t[j]
            q, v = _quantize(np.array([z]), s32, z32, maxq)
            q = float(q[0])
            if forced_codes is not None:
                fq = float(forced_codes[i, j])
                if fq != q:
                    mid = 0.5 * (q + fq) - z64
                    dist = abs(float(v[0]) - mid) if abs(q - fq) == 1 else np.inf
                    mism.append((i, j, int(q), int(fq), float(dist)))
                    q = fq
            wq = s64 * (q - z64)
            codes[i, j] = int(q)
            what[i, j] = wq
            eps[i, j] = z - wq
            e[j] = (z - wq) / (uo * U_in[j, j])
            t[j + 1:] += e[j] * U_in[j, j + 1:]
        M[i] = e @ U_in
    return dict(codes=codes, what=what, eps=eps, mismatches=mism)


def quantize_two_sided(W0, U_in, U_out, bits: int, P=None, grid0=None, forced_codes=None):
    """Target, grid and rounding (readings R-Y3 and R-Y4).

    W* = W0 + W0 P (P strictly upper, the GPTAQ correction) or W0; one grid
    per row from W0 in fp32 (or ``grid0 = (scale, zero)``); then
    round_two_sided. Returns its dict plus ``scale`` and ``zero``.
    """
    W0 = np.asarray(W0, dtype=np.float64)
    Wt = W0 if P is None else W0 + W0 @ np.asarray(P, dtype=np.float64)
    if grid0 is None:
        sc, zr = grid_fp32(W0.astype(np.float32), bits)
    else:
        sc, zr = grid0
    res = round_two_sided(Wt, U_in, U_out, sc, zr, bits, forced_codes=forced_codes)
    res["scale"], res["zero"] = np.asarray(sc, np.float32), np.asarray(zr, np.float32)
    return res


def kron_objective(dW, H_in, H_out) -> float:
    """tr(dW H_in dW^T H_out) = vec(dW)^T (H_out (x) H_in) vec(dW) for
    row-major vec: the proxy objective of [YQ] "损失函数 / 训练策略"."""
    dW = np.asarray(dW, dtype=np.float64)
    return float(np.sum((dW @ np.asarray(H_in, np.float64) @ dW.T) * np.asarray(H_out, np.float64)))


def residuals_of(Wt, What, U_in, U_out):
    """Rounding residuals eps = z - w^ implied by a finished result.

    From the definition of z (round_two_sided), W* - W^ = U_out^T e U_in
    exactly (the sum over k <= i, l <= j including (i, j) itself), so
    e = U_out^-T (W* - W^) U_in^-1 by two triangular solves and
    eps_ij = e_ij U_out[i,i] U_in[j,j]. A result is the rounding of its own
    fed-back inputs exactly when every eps lies within half a grid step
    (beyond it only toward a clamped end of the grid): a check that holds at
    any size without rerunning the rounding.
    """
    from scipy.linalg import solve_triangular

    Dl = np.asarray(Wt, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    U_in = np.asarray(U_in, dtype=np.float64)
    U_out = np.asarray(U_out, dtype=np.float64)
    X = solve_triangular(U_out, Dl, trans="T", lower=False)        # U_out^T X = Dl
    e = solve_triangular(U_in, X.T, trans="T", lower=False).T      # e U_in = X
    return e * np.diag(U_out)[:, None] * np.diag(U_in)[None, :]


def rounding_violation(eps, codes, scale, bits: int):
    """Largest excess of |eps| over half a grid step, in grid steps (<= 0 for
    a valid rounding): interior codes need |eps| <= step / 2, code 0 needs
    eps <= step / 2 and the top code eps >= -step / 2."""
    sc = np.asarray(scale, dtype=np.float64).reshape(-1)[:, None]
    r = np.asarray(eps, dtype=np.float64) / sc
    q = np.asarray(codes)
    top = 2 ** bits - 1
    over = np.where(q == 0, r - 0.5, np.where(q == top, -r - 0.5, np.abs(r) - 0.5))
    return float(over.max())
