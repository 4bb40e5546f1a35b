"""fp64 reference of KronQ's per-linear-layer solver (test infrastructure only).

Notation follows the pages: a layer y = W x with W of shape d_out x d_in, H_X
the activation covariance, H_G the output-gradient covariance, Delta X the
input drift of the quantized model. In memory, token-major arrays of shape
N x d hold one token per row, so H_X = X~^T X~ / N here is E[x x^T] of the page.

Sources (cited by page and section only):
  [KS]  KronQ summary on hyper.ai, section "方法" (Method).
  [GS]  KronQ explainer on gist.science, "Riepilogo Tecnico" -> "Metodologia".

Readings where the pages are silent or garbled are marked "Reading:".
Everything is plain numpy in float64 unless a step decides an integer (the
grid), which is done in float32 as the kernel does it.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# input decoding and the bf16 drift tensor
# --------------------------------------------------------------------------


def decode_inputs(a: np.ndarray) -> np.ndarray:
    """fp32 values of an input array: uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(a, dtype=np.float32)


def bf16_rne(a32: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values.

    IEEE-754 binary32 keeps 23 fraction bits; bf16 keeps the top 7. Rounding to
    nearest-even adds 0x7FFF plus the lowest kept bit, then truncates.
    """
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return ((r << 16).astype(np.uint32)).view(np.float32)


def covariances(X, Xq, G, n_total: int | None = None):
    """H_X, D = Delta X^T X~ / N and H_G from token-major calibration data.

    [KS] Method, Fisher equation and the K-FAC step: H ~ H_X (x) H_G with
    H_X = E[x x^T], H_G = E[g g^T]; [KS] Method, GPTAQ objective: the asymmetric
    term Delta X X^T.
    Reading: H_X is built from the quantized model's input X~ and
    Delta X = X - X~ (expanding ||W X - W^ X~||^2 gives H_X = X~ X~^T and the
    cross term W Delta X X~^T Delta W^T with a factor 2). For bf16 inputs the
    drift is itself a bf16 tensor: the fp32 difference rounded to nearest-even.
    Any of X, Xq, G may be None.
    """
    n = None
    HX = D = HG = None
    if Xq is not None:
        xq32 = decode_inputs(Xq)
        n = xq32.shape[0] if n_total is None else n_total
        xq = xq32.astype(np.float64)
        HX = xq.T @ xq / n
        if X is not None:
            x32 = decode_inputs(X)
            d32 = (x32 - xq32).astype(np.float32)
            if X.dtype == np.uint16:
                d32 = bf16_rne(d32)
            D = d32.astype(np.float64).T @ xq / n
    if G is not None:
        g = decode_inputs(G).astype(np.float64)
        ng = g.shape[0] if n_total is None else n_total
        HG = g.T @ g / ng
    return HX, D, HG


# --------------------------------------------------------------------------
# bidirectional incoherence processing
# --------------------------------------------------------------------------


def sylvester(b: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix of order b (a power of two)."""
    if b < 1 or b & (b - 1):
        raise ValueError("order must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < b:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_block(d: int) -> int:
    """Largest power of two dividing d (the blockwise rule for non-power-of-two sizes)."""
    return d & (-d)


def hadamard_rows(rows, sign: np.ndarray, b: int) -> np.ndarray:
    """Dense rows ``rows`` of V = blockdiag(H_b / sqrt(b), ...) @ diag(sign).

    Entry (r, c) of the Sylvester matrix is (-1)^popcount(r & c); row i of V
    is nonzero only on its own block. For checks of single entries of
    V M V^T without forming the whole transform.
    """
    sign = np.asarray(sign, dtype=np.float64)
    d = sign.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], d))
    c = np.arange(b, dtype=np.int64)
    for k, i in enumerate(rows):
        blk = (int(i) // b) * b
        bits = np.bitwise_and(int(i) - blk, c)
        par = np.zeros(b, dtype=np.int64)
        while np.any(bits):
            par ^= bits & 1
            bits >>= 1
        out[k, blk:blk + b] = (1 - 2 * par) * sign[blk:blk + b] / np.sqrt(b)
    return out


def apply_hadamard_left(M: np.ndarray, sign: np.ndarray, b: int) -> np.ndarray:
    """V @ M with V = blockdiag(H_b / sqrt(b), ...) @ diag(sign).

    Reading: the random Hadamard of [KS] Method (rotation step) is random signs
    followed by a normalised Sylvester transform, applied blockwise with b the
    largest power of two dividing the dimension.
    """
    d = M.shape[0]
    if d % b:
        raise ValueError("block must divide the dimension")
    hb = sylvester(b) / np.sqrt(b)
    sm = np.asarray(sign, dtype=np.float64)[:, None] * M
    out = np.empty_like(sm)
    for k in range(d // b):
        out[k * b:(k + 1) * b] = hb @ sm[k * b:(k + 1) * b]
    return out


def apply_hadamard_right(M: np.ndarray, sign: np.ndarray, b: int) -> np.ndarray:
    """M @ V^T, i.e. (V @ M^T)^T."""
    return apply_hadamard_left(M.T, sign, b).T


def _quarter_scale(diag_h: np.ndarray, sq_norm: np.ndarray) -> np.ndarray:
    """(diag(H) / ||w||^2)^(1/4); reading: a zero diagonal or zero norm gives 1."""
    out = np.ones_like(diag_h, dtype=np.float64)
    ok = (diag_h > 0) & (sq_norm > 0)
    out[ok] = (diag_h[ok] / sq_norm[ok]) ** 0.25
    return out


def biip(W, HX, D, HG, sign_in, sign_out, blk_in: int = 0, blk_out: int = 0):
    """Bidirectional incoherence processing.

    [KS] Method, BiIP scaling equation: W <- S_G W S_X with
    S_X = diag([H_X]_jj / ||W_:,j||^2)^(1/4) and S_G = diag([H_G]_ii / ||W_i,:||^2)^(1/4);
    then the rotation equation: W <- U W V^T, H_X <- V H_X V^T,
    H_G <- U H_G U^T, Delta X X^T <- V Delta X X^T V^T, with U and V random
    Hadamard transforms. [GS] Metodologia, BiIP.
    Reading: both scalings use the unscaled W; the covariances take the
    inverse scalings (H_X <- S_X^-1 H_X S_X^-1, same for the drift term,
    H_G <- S_G^-1 H_G S_G^-1) so that tr[H_G dW H_X dW^T] is unchanged.
    Returns W', H_X', D', H_G', s_x (= diag S_X), s_g (= diag S_G).
    """
    W = np.asarray(W, dtype=np.float64)
    d_out, d_in = W.shape
    bi = blk_in or hadamard_block(d_in)
    bo = blk_out or hadamard_block(d_out)
    c = np.sum(W * W, axis=0)
    r = np.sum(W * W, axis=1)
    s_x = _quarter_scale(np.diag(HX).astype(np.float64), c)
    s_g = _quarter_scale(np.diag(HG).astype(np.float64), r)
    W1 = s_g[:, None] * W * s_x[None, :]
    HX1 = np.asarray(HX, np.float64) / np.outer(s_x, s_x)
    HG1 = np.asarray(HG, np.float64) / np.outer(s_g, s_g)
    W2 = apply_hadamard_right(apply_hadamard_left(W1, sign_out, bo), sign_in, bi)
    HX2 = apply_hadamard_right(apply_hadamard_left(HX1, sign_in, bi), sign_in, bi)
    HG2 = apply_hadamard_right(apply_hadamard_left(HG1, sign_out, bo), sign_out, bo)
    D2 = None
    if D is not None:
        D1 = np.asarray(D, np.float64) / np.outer(s_x, s_x)
        D2 = apply_hadamard_right(apply_hadamard_left(D1, sign_in, bi), sign_in, bi)
    return W2, HX2, D2, HG2, s_x, s_g


def sensitivity(HX, HG):
    """s = tr(H_G) * tr(H_X), taken after BiIP and before damping.

    [KS] Method, sensitivity definition (expected loss proportional to the
    product of the two traces); [GS] Metodologia, mixed-precision metric.
    Returns (tr H_X, tr H_G, s).
    """
    tx = float(np.trace(np.asarray(HX, np.float64)))
    tg = float(np.trace(np.asarray(HG, np.float64)))
    return tx, tg, tx * tg


def covariance_diagonals(Xq, G, n_total: int | None = None):
    """diag(H_X) and diag(H_G) alone: sum over tokens of x~_j^2 (g_i^2) / N.

    The diagonals of the covariances in covariances(), without the O(N d^2)
    products, for layers too wide for the full fp64 matrices on a host.
    """
    dx = dg = None
    if Xq is not None:
        xq = decode_inputs(Xq).astype(np.float64)
        n = xq.shape[0] if n_total is None else n_total
        dx = np.einsum("tj,tj->j", xq, xq) / n
    if G is not None:
        g = decode_inputs(G).astype(np.float64)
        n = g.shape[0] if n_total is None else n_total
        dg = np.einsum("ti,ti->i", g, g) / n
    return dx, dg


def biip_scales(diag_hx, W, diag_hg):
    """(s_x, s_g): the BiIP scalings of [KS] Method from the diagonals and W."""
    W = np.asarray(W, dtype=np.float64)
    return (_quarter_scale(np.asarray(diag_hx, np.float64), np.sum(W * W, axis=0)),
            _quarter_scale(np.asarray(diag_hg, np.float64), np.sum(W * W, axis=1)))


def scaled_traces(diag_hx, W, diag_hg):
    """(tr H_X', tr H_G', s) from the diagonals and W, without forming BiIP.

    [KS] Method, BiIP: the scaling takes H_X to S_X^-1 H_X S_X^-1 (reading of
    biip()), whose trace is sum_j [H_X]_jj / s_j^2; the Hadamard rotation is
    orthogonal and leaves the trace unchanged. Same on the output side. The
    sensitivity is the product ([KS] Method, sensitivity).
    """
    dhx = np.asarray(diag_hx, np.float64)
    dhg = np.asarray(diag_hg, np.float64)
    s_x, s_g = biip_scales(dhx, W, dhg)
    tx = float(np.sum(dhx / (s_x * s_x)))
    tg = float(np.sum(dhg / (s_g * s_g)))
    return tx, tg, tx * tg


# --------------------------------------------------------------------------
# inverse-Hessian factor and the asymmetric correction
# --------------------------------------------------------------------------


def damped(H, damp: float) -> np.ndarray:
    """H + damp * mean(diag H) * I (the workloads' 1% damping)."""
    H = np.asarray(H, np.float64)
    return H + damp * np.mean(np.diag(H)) * np.eye(H.shape[0])


def inv_factor(H, damp: float) -> np.ndarray:
    """Upper-triangular U with U^T U = (H + delta I)^-1.

    [KS] Method, column-wise OBS update: the update row [H_X^-1]_{p, p+1:} is
    read as the Cholesky form of the OBS row, i.e. U_pp * U_{p,F} equals row p
    of the inverse of the trailing block H_{p:, p:}.
    Definition written out: invert the damped matrix, then take its Cholesky
    factor (lower L with L L^T = H^-1, U = L^T). Raises LinAlgError if the
    damped matrix is not positive definite.
    """
    Hd = damped(H, damp)
    np.linalg.cholesky(Hd)  # raises if not positive definite
    Hinv = np.linalg.inv(Hd)
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


def form_p(D, U) -> np.ndarray:
    """Asymmetric correction P = triu_1(D U^T) U (strictly upper).

    [KS] Method, OBS update equation: P is the "GPTAQ asymmetric correction"
    and is not written out on the pages. Reading: row p of P equals
    D_{p,F} (H_{FF})^-1 with F = {p+1, ...}: the least-squares compensation, by
    the still-free columns, of the drift of the column just fixed. With
    U^T U = H^-1 this is the strictly upper part of D U^T, times U.
    """
    T = np.triu(np.asarray(D, np.float64) @ np.asarray(U, np.float64).T, 1)
    return T @ np.asarray(U, np.float64)


def form_p_rows(D_rows, rows, U) -> np.ndarray:
    """Rows ``rows`` of P = triu_1(D U^T) U, from the same rows of D.

    Row p of P needs row p of D only: t = D_p U^T with t_k = 0 for k <= p,
    then t U (the definition of form_p() restricted to some rows).
    """
    U = np.asarray(U, dtype=np.float64)
    T = np.asarray(D_rows, dtype=np.float64) @ U.T
    n = U.shape[0]
    k = np.arange(n)
    for r, p in enumerate(np.asarray(rows, dtype=np.int64)):
        T[r, k <= p] = 0.0
    return T @ U


# --------------------------------------------------------------------------
# grid and the column sweep
# --------------------------------------------------------------------------


def grid_fp32(rows: np.ndarray, bits: int):
    """Asymmetric min-max grid per row, computed in fp32 as the kernel does.

    [KS] Method and experiments: uniform 2/3/4-bit weight-only grids, per
    output channel or per group of 128 columns.
    Reading (GPTQ-family min-max quantizer): lo = min(row, 0), hi = max(row, 0),
    an all-zero row takes [-1, 1]; scale = (hi - lo) / (2^b - 1) and
    zero = rint(-lo / scale), rint rounding half to even. Returns fp32 arrays.
    """
    v = np.asarray(rows, dtype=np.float32)
    maxq = np.float32(2 ** bits - 1)
    lo = np.minimum(v.min(axis=1), np.float32(0))
    hi = np.maximum(v.max(axis=1), np.float32(0))
    same = lo == hi
    lo = np.where(same, np.float32(-1), lo).astype(np.float32)
    hi = np.where(same, np.float32(1), hi).astype(np.float32)
    scale = ((hi - lo).astype(np.float32) / maxq).astype(np.float32)
    zero = np.rint((-lo).astype(np.float32) / scale).astype(np.float32)
    return scale, zero


def _quantize(w, scale, zero, maxq):
    """Code and pre-rounding value of w on the grid (scale, zero)."""
    v = w / scale.astype(np.float64)
    q = np.clip(np.rint(v) + zero.astype(np.float64), 0, maxq)
    return q, v


def sweep(W0, U, P, bits: int, group: int = 0, block: int = 128,
          forced_codes=None, forced_grid=None, grid0=None, trace=None):
    """Blocked GPTAQ column sweep (lazy batch updates of ``block`` columns).

    [KS] Method, OBS update: after quantizing column p,
        Delta W_{:, p+1:} = -delta_p [H_X^-1]_{p, p+1:} + W_{:, p} P_{p, p+1:}
    Reading: delta_p = (w_p - w^_p) / U_pp with w_p the working column, the
    inverse row is row p of U, and W_{:, p} is the original (post-BiIP) W0.
    H_G does not enter ([GS] Metodologia, Proposition 1). Updates to columns
    of later blocks are accumulated and applied at the end of each block, as
    the lazy-batch form of the sweep does; ``block >= d_in`` is the unblocked
    form. Per-channel grids come from W0 (or ``grid0``); group grids are taken
    when the sweep reaches the group's first column, from the working values
    rounded to fp32 (``group`` must divide ``block``).

    Forced replay: if ``forced_codes`` (d_out x d_in) is given, each code that
    differs from the oracle's is recorded with the distance of the oracle's
    pre-rounding value to the midpoint between the two codes (in grid steps),
    then the forced code is adopted so that one legitimate flip does not
    cascade along the row. ``forced_grid = (scale, zero)`` (d_out x n_groups)
    does the same for group grids. ``trace(p, W)``, if given, is called after
    column p with the working matrix (for checks of intermediate states).

    Returns dict(codes uint8, what float64, scale, zero, mismatches list of
    (row, col, oracle_code, forced_code, midpoint_distance), grid_mismatch).
    """
    W0 = np.asarray(W0, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    P = None if P is None else np.asarray(P, dtype=np.float64)
    d_out, n = W0.shape
    if group and block % group:
        raise ValueError("group must divide block")
    maxq = 2 ** bits - 1
    W = W0.copy()
    codes = np.zeros((d_out, n), dtype=np.uint8)
    what = np.zeros((d_out, n))
    n_groups = (n + group - 1) // group if group else 1
    scales = np.zeros((d_out, n_groups), dtype=np.float32)
    zeros = np.zeros((d_out, n_groups), dtype=np.float32)
    mism = []
    grid_mism = []
    if not group:
        if grid0 is not None:
            sc, zr = grid0
        else:
            sc, zr = grid_fp32(W0.astype(np.float32), bits)
        scales[:, 0], zeros[:, 0] = sc, zr
    for b0 in range(0, n, block):
        b1 = min(b0 + block, n)
        E = np.zeros((d_out, b1 - b0))
        for p in range(b0, b1):
            g = p // group if group else 0
            if group and p % group == 0:
                sc, zr = grid_fp32(W[:, p:min(p + group, n)].astype(np.float32), bits)
                if forced_grid is not None:
                    fs = np.asarray(forced_grid[0])[:, g].astype(np.float32)
                    fz = np.asarray(forced_grid[1])[:, g].astype(np.float32)
                    grid_mism.append((np.max(np.abs(fs / sc - 1)), int(np.sum(fz != zr))))
                    sc, zr = fs, fz
                scales[:, g], zeros[:, g] = sc, zr
            sc = scales[:, g]
            zr = zeros[:, g]
            w = W[:, p]
            q, v = _quantize(w, sc, zr, maxq)
            if forced_codes is not None:
                fq = np.asarray(forced_codes[:, p], dtype=np.float64)
                bad = np.nonzero(fq != q)[0]
                for i in bad:
                    # midpoint between the two codes, in pre-rounding units
                    mid = 0.5 * (q[i] + fq[i]) - zr[i]
                    dist = abs(v[i] - mid) if abs(q[i] - fq[i]) == 1 else np.inf
                    mism.append((int(i), p, int(q[i]), int(fq[i]), float(dist)))
                q = fq
            wq = sc.astype(np.float64) * (q - zr.astype(np.float64))
            codes[:, p] = q.astype(np.uint8)
            what[:, p] = wq
            e = (w - wq) / U[p, p]
            E[:, p - b0] = e
            if p + 1 < b1:
                W[:, p + 1:b1] -= np.outer(e, U[p, p + 1:b1])
                if P is not None:
                    W[:, p + 1:b1] += np.outer(W0[:, p], P[p, p + 1:b1])
            if trace is not None:
                trace(p, W)
        if b1 < n:
            W[:, b1:] -= E @ U[b0:b1, b1:]
            if P is not None:
                W[:, b1:] += W0[:, b0:b1] @ P[b0:b1, b1:]
    return dict(codes=codes, what=what, scale=scales, zero=zeros,
                mismatches=mism, grid_mismatch=grid_mism)


def rtn(W0, bits: int, group: int = 0):
    """Round-to-nearest on the same grid, every entry rounded on its own."""
    W0 = np.asarray(W0, dtype=np.float64)
    d_out, n = W0.shape
    maxq = 2 ** bits - 1
    codes = np.zeros((d_out, n), dtype=np.uint8)
    what = np.zeros((d_out, n))
    gs = group or n
    for g0 in range(0, n, gs):
        g1 = min(g0 + gs, n)
        sc, zr = grid_fp32(W0[:, g0:g1].astype(np.float32), bits)
        q, _ = _quantize(W0[:, g0:g1], sc[:, None], zr[:, None], maxq)
        codes[:, g0:g1] = q.astype(np.uint8)
        what[:, g0:g1] = sc[:, None].astype(np.float64) * (q - zr[:, None].astype(np.float64))
    return codes, what


# --------------------------------------------------------------------------
# objective, diagnostics, allocation
# --------------------------------------------------------------------------


def objective(W0, What, HX, D, HG) -> float:
    """tr[H_G (dW H_X dW^T + 2 W0 D dW^T)] with dW = W0 - W^.

    [KS] Method, Kronecker objective tr[H_G dW H_X dW^T] and its GPTAQ
    extension with the drift term. Reading: the drift term carries the factor
    2 from expanding the square and a plus sign with D = Delta X X~^T / N,
    Delta X = X - X~; D = None gives the plain Kronecker objective.
    """
    W0 = np.asarray(W0, np.float64)
    dW = W0 - np.asarray(What, np.float64)
    M = dW @ np.asarray(HX, np.float64)
    if D is not None:
        M = M + 2.0 * (W0 @ np.asarray(D, np.float64))
    K = M @ dW.T
    return float(np.sum(np.asarray(HG, np.float64) * K.T))


def mu_incoherence(H) -> float:
    """mu(H) / sqrt(d) = max_ij |Q_ij| for H = Q Lambda Q^T.

    [KS] Method, incoherence measure mu(H_G)/sqrt(d_out) (not defined on the
    pages). Reading: QuIP's incoherence of the eigenvector matrix.
    """
    _, Q = np.linalg.eigh(np.asarray(H, np.float64))
    return float(np.max(np.abs(Q)))


def cv_in_out(W):
    """(CV_in, CV_out): std/mean of the column norms and of the row norms.

    [KS] Method, BiIP discussion of the coefficients of variation of the
    weight magnitudes along the input and output dimensions.
    """
    W = np.asarray(W, np.float64)
    cn = np.sqrt(np.sum(W * W, axis=0))
    rn = np.sqrt(np.sum(W * W, axis=1))
    return float(np.std(cn) / np.mean(cn)), float(np.std(rn) / np.mean(rn))


def allocate_bits(s, n_params, widths=(2, 3, 4), avg_budget: float = 2.5):
    """Mixed-precision widths by descending sensitivity under an average budget.

    [KS] Method, sensitivity ranking: sublayers with larger s get more bits.
    Reading: visit sublayers in descending s (ties by input order) and give
    each the widest width that still leaves every unvisited sublayer its
    narrowest width within sum(b * n) <= avg_budget * sum(n).
    """
    s = np.asarray(s, dtype=np.float64)
    n = np.asarray(n_params, dtype=np.float64)
    ws = sorted(widths)
    wmin = ws[0]
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    budget = avg_budget * float(np.sum(n))
    used = wmin * float(np.sum(n))
    if used > budget:
        raise ValueError("budget below the narrowest width")
    bits = [wmin] * len(s)
    for i in order:
        for w in reversed(ws):
            extra = (w - wmin) * n[i]
            if used + extra <= budget:
                bits[i] = w
                used += extra
                break
    return bits


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------


def quantize_layer(X, Xq, G, W, sign_in, sign_out, bits: int, group: int = 0,
                   block: int = 128, damp: float = 0.01, n_total=None):
    """Covariances -> BiIP -> sensitivity -> damped inverse factor -> P -> sweep.

    Returns a dict with every intermediate (all float64) plus the objective of
    the sweep and of round-to-nearest on the processed problem.
    """
    HX, D, HG = covariances(X, Xq, G, n_total)
    return solve_layer(HX, D, HG, W, sign_in, sign_out, bits, group, block, damp)


def covariances_chunked(token_chunks, n_total: int):
    """covariances() summed over an iterable of (X, Xq, G) token chunks.

    The covariances are sums over tokens, so a layer with more tokens than a
    host holds at once in fp64 is accumulated a chunk at a time.
    """
    HX = D = HG = None
    for X, Xq, G in token_chunks:
        parts = covariances(X, Xq, G, n_total)
        HX, D, HG = [p if acc is None else (acc if p is None else acc + p)
                     for acc, p in zip((HX, D, HG), parts)]
    return HX, D, HG


def solve_layer(HX, D, HG, W, sign_in, sign_out, bits: int, group: int = 0,
                block: int = 128, damp: float = 0.01):
    """Everything after the covariances: BiIP -> sensitivity -> damped inverse
    factor -> P -> sweep, with the objective of the sweep and of
    round-to-nearest on the processed problem (see quantize_layer)."""
    W2, HX2, D2, HG2, s_x, s_g = biip(W, HX, D, HG, sign_in, sign_out)
    tx, tg, s = sensitivity(HX2, HG2)
    U = inv_factor(HX2, damp)
    P = form_p(D2, U)
    res = sweep(W2, U, P, bits, group, block)
    codes_rtn, what_rtn = rtn(W2, bits, group)
    return dict(HX=HX, D=D, HG=HG, W2=W2, HX2=HX2, D2=D2, HG2=HG2, s_x=s_x, s_g=s_g,
                trHX=tx, trHG=tg, s=s, U=U, P=P, codes=res["codes"], what=res["what"],
                scale=res["scale"], zero=res["zero"],
                obj=objective(W2, res["what"], HX2, D2, HG2),
                obj_rtn=objective(W2, what_rtn, HX2, D2, HG2), codes_rtn=codes_rtn)
