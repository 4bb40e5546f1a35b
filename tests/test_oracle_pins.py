"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check uses a closed form,
brute force over tiny inputs, a library routine, or a value worked by hand
(``tests/golden``). A plausible slip in the oracle (a dropped term, a wrong
sign or index, a transposed operand) fails at least one of them.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from synth import layer_specs, make_layer

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _spd(rng, n, cond=10.0):
    q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    ev = np.exp(rng.uniform(0, np.log(cond), n))
    return (q * ev) @ q.T


def _dyadic(rng, shape, scale=8):
    """Values k/64 with |k| small: fp32 sums and differences of these are exact."""
    return (rng.integers(-scale * 64, scale * 64, shape) / 64.0).astype(np.float32)


# --------------------------------------------------------------------------- bf16


def _bf16_by_frexp(x):
    """Nearest-even bf16 via the significand: 8 significant bits, rint = ties to even."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def test_bf16_rne_golden():
    for case in _load("bf16_rne.json")["cases"]:
        f = np.array([int(case["f32_bits"], 16)], dtype=np.uint32).view(np.float32)
        want = (np.array([int(case["bf16_bits"], 16)], dtype=np.uint32) << 16).view(np.float32)
        got = oracle.bf16_rne(f)
        assert got.view(np.uint32)[0] == want.view(np.uint32)[0], case["why"]


def test_bf16_rne_matches_significand_rounding():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # include exact ties
    ties = (np.float32(1.0) + np.arange(1, 255, 2, dtype=np.float32) * np.float32(2.0 ** -8))
    x = np.concatenate([x, ties, -ties])
    np.testing.assert_array_equal(oracle.bf16_rne(x).astype(np.float64), _bf16_by_frexp(x))


# --------------------------------------------------------------------- covariances


@pytest.mark.parametrize("bf16", [False, True])
def test_covariances_against_token_loop(bf16):
    rng = np.random.default_rng(2)
    n, d_in, d_out = 24, 5, 3
    x = rng.standard_normal((n, d_in)).astype(np.float32)
    xq = (x + 0.01 * rng.standard_normal((n, d_in))).astype(np.float32)
    g = rng.standard_normal((n, d_out)).astype(np.float32)
    if bf16:
        to16 = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 values do
        X, Xq, G = to16(x), to16(xq), to16(g)
        xv = (X.astype(np.uint32) << 16).view(np.float32)
        xqv = (Xq.astype(np.uint32) << 16).view(np.float32)
        gv = (G.astype(np.uint32) << 16).view(np.float32)
    else:
        X, Xq, G = x, xq, g
        xv, xqv, gv = x, xq, g
    HX, D, HG = oracle.covariances(X, Xq, G)
    hx = np.zeros((d_in, d_in))
    dd = np.zeros((d_in, d_in))
    hg = np.zeros((d_out, d_out))
    for t in range(n):
        a = xqv[t].astype(np.float64)
        delta = np.float32(xv[t]) - np.float32(xqv[t])
        if bf16:
            delta = _bf16_by_frexp(delta.astype(np.float32))
        delta = np.asarray(delta, np.float64)
        gg = gv[t].astype(np.float64)
        for i in range(d_in):
            for j in range(d_in):
                hx[i, j] += a[i] * a[j] / n
                dd[i, j] += delta[i] * a[j] / n
        for i in range(d_out):
            for j in range(d_out):
                hg[i, j] += gg[i] * gg[j] / n
    np.testing.assert_allclose(HX, hx, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(D, dd, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(HG, hg, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------- objective


def test_covariances_chunked_equal_whole():
    """The covariances are sums over tokens: chunking the stream changes nothing."""
    rng = np.random.default_rng(21)
    X = _dyadic(rng, (96, 8))
    Xq = _dyadic(rng, (96, 8))
    G = _dyadic(rng, (96, 5))
    whole = oracle.covariances(X, Xq, G)
    parts = oracle.covariances_chunked(((X[c:c + 40], Xq[c:c + 40], G[c:c + 40])
                                        for c in range(0, 96, 40)), 96)
    for w, p in zip(whole, parts):
        np.testing.assert_allclose(p, w, rtol=1e-13, atol=0)
    # the diagonals alone, chunk by chunk, divide by the whole stream's count
    dx = dg = 0.0
    for c in range(0, 96, 40):
        a, b = oracle.covariance_diagonals(Xq[c:c + 40], G[c:c + 40], 96)
        dx, dg = dx + a, dg + b
    np.testing.assert_allclose(dx, np.diag(whole[0]), rtol=1e-13, atol=0)
    np.testing.assert_allclose(dg, np.diag(whole[2]), rtol=1e-13, atol=0)


def test_kronecker_vec_identity():
    """tr[H_G dW H_X dW^T] = vec(dW)^T (H_X kron H_G) vec(dW), vec column-major."""
    rng = np.random.default_rng(3)
    d_out, d_in = 3, 4
    HX, HG = _spd(rng, d_in), _spd(rng, d_out)
    W0 = rng.standard_normal((d_out, d_in))
    Wh = rng.standard_normal((d_out, d_in))
    v = (W0 - Wh).flatten(order="F")
    want = v @ np.kron(HX, HG) @ v
    assert oracle.objective(W0, Wh, HX, None, HG) == pytest.approx(want, rel=1e-12)
    # the per-sample Fisher identity vec(g x^T) = x kron g behind it
    x, g = rng.standard_normal(d_in), rng.standard_normal(d_out)
    np.testing.assert_allclose(np.outer(g, x).flatten(order="F"), np.kron(x, g))


def test_objective_equals_expanded_residual():
    """objective = tr[H_G R R^T]/N - const, R = W0 X - W^ X~ (the GPTAQ residual)."""
    rng = np.random.default_rng(4)
    n, d_in, d_out = 40, 6, 3
    x = _dyadic(rng, (n, d_in))
    xq = (x + _dyadic(rng, (n, d_in), 1) / 8).astype(np.float32)
    g = rng.standard_normal((n, d_out)).astype(np.float32)
    HX, D, HG = oracle.covariances(x, xq, g)
    W0 = rng.standard_normal((d_out, d_in))
    Wh = W0 + 0.1 * rng.standard_normal((d_out, d_in))
    X, XQ = x.astype(np.float64), xq.astype(np.float64)
    R = X @ W0.T - XQ @ Wh.T                   # token-major residual, N x d_out
    C = (X - XQ) @ W0.T                        # the part that does not depend on W^
    want = np.trace(HG @ (R.T @ R - C.T @ C)) / n
    got = oracle.objective(W0, Wh, HX, D, HG)
    assert got == pytest.approx(want, rel=1e-10)


# --------------------------------------------------------------------- Hadamard


def test_sylvester_matches_scipy():
    for k in range(0, 10):
        np.testing.assert_array_equal(oracle.sylvester(2 ** k), scipy.linalg.hadamard(2 ** k))


def test_hadamard_blockwise_dense_and_orthogonal():
    rng = np.random.default_rng(5)
    d, b = 12, 4
    assert oracle.hadamard_block(12) == 4
    assert oracle.hadamard_block(11008) == 256 and oracle.hadamard_block(28672) == 4096
    sign = rng.choice([-1, 1], d)
    V = np.kron(np.eye(d // b), scipy.linalg.hadamard(b) / np.sqrt(b)) @ np.diag(sign)
    M = rng.standard_normal((d, 7))
    np.testing.assert_allclose(oracle.apply_hadamard_left(M, sign, b), V @ M, atol=1e-13)
    N = rng.standard_normal((5, d))
    np.testing.assert_allclose(oracle.apply_hadamard_right(N, sign, b), N @ V.T, atol=1e-13)
    np.testing.assert_allclose(V @ V.T, np.eye(d), atol=1e-12)
    Vm = oracle.apply_hadamard_left(np.eye(d), sign, b)
    np.testing.assert_allclose(Vm.T @ Vm, np.eye(d), atol=1e-12)


# ------------------------------------------------------------------------ BiIP


def _small_problem(seed=6, n=64, d_in=16, d_out=8):
    rng = np.random.default_rng(seed)
    sig = np.exp(rng.standard_normal(d_in))
    sig[:2] *= 20
    tau = np.exp(2 * rng.standard_normal(d_out))
    x = (rng.standard_normal((n, d_in)) * sig).astype(np.float32)
    xq = (x + 0.01 * sig * rng.standard_normal((n, d_in))).astype(np.float32)
    g = (rng.standard_normal((n, d_out)) * tau).astype(np.float32)
    W = 0.02 * rng.standard_normal((d_out, d_in))
    si = rng.choice([-1, 1], d_in)
    so = rng.choice([-1, 1], d_out)
    return x, xq, g, W, si, so


def test_biip_closed_form_traces_and_sensitivity():
    x, xq, g, W, si, so = _small_problem()
    HX, D, HG = oracle.covariances(x, xq, g)
    W2, HX2, D2, HG2, s_x, s_g = oracle.biip(W, HX, D, HG, si, so)
    c = np.sum(W * W, axis=0)
    r = np.sum(W * W, axis=1)
    trx = np.sum(np.sqrt(np.diag(HX) * c))
    trg = np.sum(np.sqrt(np.diag(HG) * r))
    assert np.trace(HX2) == pytest.approx(trx, rel=1e-12)
    assert np.trace(HG2) == pytest.approx(trg, rel=1e-12)
    tx, tg, s = oracle.sensitivity(HX2, HG2)
    assert s == pytest.approx(trx * trg, rel=1e-12)
    # scales straight from the scaling equation
    np.testing.assert_allclose(s_x, (np.diag(HX) / c) ** 0.25, rtol=1e-13)
    np.testing.assert_allclose(s_g, (np.diag(HG) / r) ** 0.25, rtol=1e-13)


def test_diagonal_shortcuts_match_full_forms():
    """covariance_diagonals / scaled_traces (used where the full fp64 matrices
    do not fit a host) agree with the full covariances, BiIP and traces."""
    x, xq, g, W, si, so = _small_problem()
    HX, D, HG = oracle.covariances(x, xq, g)
    dx, dg = oracle.covariance_diagonals(xq, g)
    np.testing.assert_allclose(dx, np.diag(HX), rtol=1e-13)
    np.testing.assert_allclose(dg, np.diag(HG), rtol=1e-13)
    W2, HX2, D2, HG2, s_x, s_g = oracle.biip(W, HX, D, HG, si, so)
    tx, tg, s = oracle.scaled_traces(dx, W, dg)
    assert tx == pytest.approx(np.trace(HX2), rel=1e-12)
    assert tg == pytest.approx(np.trace(HG2), rel=1e-12)
    assert s == pytest.approx(oracle.sensitivity(HX2, HG2)[2], rel=1e-12)
    # a zero column of W leaves its diagonal entry unscaled
    W0 = W.copy()
    W0[:, 3] = 0
    tx0, _, _ = oracle.scaled_traces(dx, W0, dg)
    c = np.sum(W0 * W0, axis=0)
    want = np.sum(np.where(c > 0, np.sqrt(dx * c), dx))
    assert tx0 == pytest.approx(want, rel=1e-12)


def test_row_forms_match_whole_matrix_forms():
    """hadamard_rows and form_p_rows (single-entry checks at full size) agree
    with the dense Sylvester construction and with form_p."""
    rng = np.random.default_rng(21)
    for d, b in ((48, 16), (64, 64), (40, 8)):
        sign = rng.choice([-1, 1], d)
        Vd = oracle.apply_hadamard_left(np.eye(d), sign, b)
        rows = rng.choice(d, 7, replace=False)
        np.testing.assert_array_equal(oracle.hadamard_rows(rows, sign, b), Vd[rows])
    n = 96
    H = _spd(rng, n)
    U = oracle.inv_factor(H, 0.01)
    D = rng.standard_normal((n, n))
    rows = np.array([0, 5, 47, 94, 95])
    np.testing.assert_allclose(oracle.form_p_rows(D[rows], rows, U), oracle.form_p(D, U)[rows],
                               rtol=1e-12, atol=1e-12)
    x, xq, g, W, si, so = _small_problem()
    HX, D, HG = oracle.covariances(x, xq, g)
    _, _, _, _, s_x, s_g = oracle.biip(W, HX, D, HG, si, so)
    bx, bg = oracle.biip_scales(np.diag(HX), W, np.diag(HG))
    np.testing.assert_array_equal(bx, s_x)
    np.testing.assert_array_equal(bg, s_g)


def test_biip_rotation_preserves_traces():
    rng = np.random.default_rng(7)
    M = _spd(rng, 16)
    s = rng.choice([-1, 1], 16)
    R = oracle.apply_hadamard_right(oracle.apply_hadamard_left(M, s, 16), s, 16)
    assert np.trace(R) == pytest.approx(np.trace(M), rel=1e-13)
    np.testing.assert_allclose(np.linalg.eigvalsh(R), np.linalg.eigvalsh(M), rtol=1e-11)


def test_biip_objective_invariant():
    """tr[H_G dW H_X dW^T] and the drift term are unchanged by BiIP."""
    x, xq, g, W, si, so = _small_problem()
    HX, D, HG = oracle.covariances(x, xq, g)
    W2, HX2, D2, HG2, s_x, s_g = oracle.biip(W, HX, D, HG, si, so)
    rng = np.random.default_rng(8)
    Wh = W + 0.005 * rng.standard_normal(W.shape)
    Wh1 = s_g[:, None] * Wh * s_x[None, :]
    Wh2 = oracle.apply_hadamard_right(oracle.apply_hadamard_left(Wh1, so, 8), si, 16)
    a = oracle.objective(W, Wh, HX, D, HG)
    b = oracle.objective(W2, Wh2, HX2, D2, HG2)
    assert b == pytest.approx(a, rel=1e-10)


def test_biip_incoherence_and_cv_drop():
    """mu(H_G)/sqrt(d_out) falls; the output rotation lowers CV_out while an
    input-only rotation leaves the row norms (hence CV_out) exactly unchanged."""
    spec = layer_specs(0)[0]
    L = make_layer(spec)
    HX, D, HG = oracle.covariances(L["x"], L["xq"], L["g"])
    W2, HX2, D2, HG2, s_x, s_g = oracle.biip(L["W"], HX, D, HG, L["sign_in"], L["sign_out"])
    mu0 = oracle.mu_incoherence(HG)
    mu1 = oracle.mu_incoherence(HG2)
    assert mu0 > 0.9 and mu1 < 0.5 * mu0
    W1 = s_g[:, None] * L["W"].astype(np.float64) * s_x[None, :]
    in_only = oracle.apply_hadamard_right(W1, L["sign_in"], 256)
    np.testing.assert_allclose(np.linalg.norm(in_only, axis=1), np.linalg.norm(W1, axis=1), rtol=1e-12)
    cvi1, cvo1 = oracle.cv_in_out(W1)
    cvi2, cvo2 = oracle.cv_in_out(W2)
    assert cvo2 < cvo1 and cvi2 < cvi1


def test_mu_special_cases():
    d = 16
    Hd = np.diag(np.arange(1.0, d + 1))
    assert oracle.mu_incoherence(Hd) == pytest.approx(1.0)
    Q = scipy.linalg.hadamard(d) / np.sqrt(d)
    assert oracle.mu_incoherence(Q @ Hd @ Q.T) == pytest.approx(1 / np.sqrt(d), rel=1e-9)


# -------------------------------------------------------- factor, P, the sweep


def test_inv_factor_definition_and_obs_rows():
    rng = np.random.default_rng(9)
    n, damp = 8, 0.01
    H = _spd(rng, n, 100.0)
    U = oracle.inv_factor(H, damp)
    Hd = H + damp * np.mean(np.diag(H)) * np.eye(n)
    np.testing.assert_allclose(np.tril(U, -1), 0, atol=0)
    np.testing.assert_allclose(U.T @ U @ Hd, np.eye(n), atol=1e-10)
    for p in range(n):
        row = np.linalg.inv(Hd[p:, p:])[0]
        np.testing.assert_allclose(U[p, p] * U[p, p:], row, rtol=1e-9, atol=1e-12)
    with pytest.raises(np.linalg.LinAlgError):
        oracle.inv_factor(-np.eye(4), 0.0)


def test_form_p_obs_identity():
    rng = np.random.default_rng(10)
    n = 9
    H = _spd(rng, n, 50.0)
    D = 0.05 * rng.standard_normal((n, n))
    U = oracle.inv_factor(H, 0.0)
    P = oracle.form_p(D, U)
    np.testing.assert_allclose(np.tril(P), 0, atol=1e-14)
    for p in range(n - 1):
        F = slice(p + 1, n)
        want = D[p, F] @ np.linalg.inv(H[F, F])
        np.testing.assert_allclose(P[p, F], want, rtol=1e-9, atol=1e-12)


def test_sweep_tracks_hg_weighted_argmin():
    """After each column the working W equals the exact minimiser of the
    remaining GPTAQ residual weighted by an arbitrary SPD H_G, solved with the
    full Kronecker system: H_G cancels (Proposition 1) and the update with U
    and P is the least-squares compensation."""
    rng = np.random.default_rng(11)
    n_tok, d_in, d_out, bits = 48, 6, 3, 2
    x = _dyadic(rng, (n_tok, d_in))
    xq = (x + _dyadic(rng, (n_tok, d_in), 1) / 4).astype(np.float32)
    HX, D, _ = oracle.covariances(x, xq, None)
    HG = _spd(rng, d_out, 30.0)
    W0 = rng.standard_normal((d_out, d_in))
    U = oracle.inv_factor(HX, 0.0)
    P = oracle.form_p(D, U)
    X, XQ = x.astype(np.float64), xq.astype(np.float64)
    states = {}
    res = oracle.sweep(W0, U, P, bits, 0, block=d_in,
                       trace=lambda p, W: states.__setitem__(p, W.copy()))
    Wh = res["what"]
    for p in range(d_in - 1):
        F = list(range(p + 1, d_in))
        # fixed part of the residual (d_out x N): quantized columns see X~, targets see X
        a = W0[:, :p + 1] @ X[:, :p + 1].T - Wh[:, :p + 1] @ XQ[:, :p + 1].T + W0[:, F] @ XQ[:, F].T
        # residual = a - Wf @ XQ_F^T ; vec (column-major) is linear in vec(Wf)
        A = np.kron(XQ[:, F], np.eye(d_out))           # vec(Wf @ XQ_F^T) = A vec(Wf)
        Wt = np.kron(np.eye(n_tok), HG)                 # tr[H_G R R^T] = vec(R)^T Wt vec(R)
        lhs = A.T @ Wt @ A
        rhs = A.T @ Wt @ a.flatten(order="F")
        wf = np.linalg.solve(lhs, rhs).reshape((d_out, len(F)), order="F")
        np.testing.assert_allclose(states[p][:, F], wf, rtol=1e-8, atol=1e-10)


def test_sweep_matches_textbook_obs_with_explicit_inverses():
    """Column loop written with explicit inverses of the trailing blocks (no
    Cholesky factor, no P matrix) gives the same codes and values."""
    rng = np.random.default_rng(12)
    d_out, n, bits, damp = 5, 10, 3, 0.01
    H = _spd(rng, n, 200.0)
    D = 0.05 * rng.standard_normal((n, n))
    W0 = rng.standard_normal((d_out, n))
    Hd = H + damp * np.mean(np.diag(H)) * np.eye(n)
    U = oracle.inv_factor(H, damp)
    res = oracle.sweep(W0, U, oracle.form_p(D, U), bits, 0, block=4)
    scale, zero = oracle.grid_fp32(W0.astype(np.float32), bits)
    W = W0.copy()
    maxq = 2 ** bits - 1
    codes = np.zeros((d_out, n), dtype=int)
    for p in range(n):
        Hi = np.linalg.inv(Hd[p:, p:])
        q = np.clip(np.rint(W[:, p] / scale) + zero, 0, maxq)
        codes[:, p] = q
        wq = scale * (q - zero)
        if p + 1 < n:
            W[:, p + 1:] -= np.outer((W[:, p] - wq) / Hi[0, 0], Hi[0, 1:])
            W[:, p + 1:] += np.outer(W0[:, p], D[p, p + 1:] @ np.linalg.inv(Hd[p + 1:, p + 1:]))
    np.testing.assert_array_equal(res["codes"], codes)


def test_sweep_reduces_to_rtn_when_hx_identity_and_no_drift():
    """With H_X = I and no drift nothing is fed back: the sweep is
    round-to-nearest, group by group, with each group's grid (a ragged last
    group included) stored in its own slot."""
    rng = np.random.default_rng(13)
    for n, group in ((64, 0), (64, 32), (104, 16)):
        W0 = rng.standard_normal((16, n)).astype(np.float32)
        U = oracle.inv_factor(np.eye(n), 0.01)
        res = oracle.sweep(W0, U, None, 2, group, block=32)
        codes, what = oracle.rtn(W0, 2, group)
        np.testing.assert_array_equal(res["codes"], codes)
        np.testing.assert_allclose(res["what"], what, rtol=0, atol=1e-15)
        gs = group or n
        for k, g0 in enumerate(range(0, n, gs)):
            sc, zr = oracle.grid_fp32(W0[:, g0:g0 + gs], 2)
            np.testing.assert_array_equal(res["scale"][:, k], sc)
            np.testing.assert_array_equal(res["zero"][:, k], zr)


def test_blocked_equals_unblocked():
    rng = np.random.default_rng(14)
    d_out, n = 12, 32
    H = _spd(rng, n, 30.0)
    D = 0.05 * rng.standard_normal((n, n))
    W0 = rng.standard_normal((d_out, n))
    U = oracle.inv_factor(H, 0.01)
    P = oracle.form_p(D, U)
    for group in (0, 8):
        ref = oracle.sweep(W0, U, P, 2, group, block=n)
        blk = oracle.sweep(W0, U, P, 2, group, block=8, forced_codes=ref["codes"])
        assert all(m[4] < 1e-9 for m in blk["mismatches"])
        np.testing.assert_allclose(blk["what"], ref["what"], atol=1e-12)


def test_forced_replay_midpoint_distance_hand_worked():
    """The replay diagnostic measures the pre-rounding value's distance to the
    midpoint between the two codes, in grid steps and relative to the zero
    point. Row [-0.25, 0.5] at 2 bits: scale 0.75/3 = 0.25, zero rint(1) = 1.
    Column 0: w/scale = -1 -> code 0; forced to 1, the midpoint of codes 0
    and 1 sits at 0.5 - 1 = -0.5 grid steps, so the distance is 0.5. Forced
    to 2 (not adjacent) the distance is infinite. With U = I nothing moves
    column 1: 0.5/0.25 = 2 -> code 3."""
    W0 = np.array([[-0.25, 0.5]])
    res = oracle.sweep(W0, np.eye(2), None, 2, 0, block=2, forced_codes=np.array([[1, 3]]))
    assert res["scale"][0, 0] == np.float32(0.25) and res["zero"][0, 0] == 1.0
    assert res["mismatches"] == [(0, 0, 0, 1, 0.5)]
    np.testing.assert_array_equal(res["codes"], [[1, 3]])
    np.testing.assert_array_equal(res["what"], [[0.0, 0.5]])
    far = oracle.sweep(W0, np.eye(2), None, 2, 0, block=2, forced_codes=np.array([[2, 3]]))
    assert far["mismatches"][0][:4] == (0, 0, 0, 2) and far["mismatches"][0][4] == np.inf


def test_solve_layer_chains_the_pinned_stages():
    """The whole-layer entry is the composition of the stages pinned above:
    the sensitivity agrees with the diagonal shortcut taken straight from the
    raw covariances and W (another route than the post-BiIP traces), each
    stored intermediate is its stage applied to the previous one, and the
    drift term reaches the sweep (dropping it changes codes here)."""
    x, xq, g, W, si, so = _small_problem(seed=9, n=256, d_in=64, d_out=16)
    HX, D, HG = oracle.covariances(x, xq, g)
    out = oracle.solve_layer(HX, D, HG, W, si, so, bits=2, group=0, block=16, damp=0.01)
    s_diag = oracle.scaled_traces(np.diag(HX), W, np.diag(HG))[2]
    assert out["s"] == pytest.approx(s_diag, rel=1e-12)
    np.testing.assert_allclose(out["U"].T @ out["U"],
                               np.linalg.inv(oracle.damped(out["HX2"], 0.01)), rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(out["P"], oracle.form_p(out["D2"], out["U"]), rtol=0, atol=0)
    with_p = oracle.sweep(out["W2"], out["U"], out["P"], 2, 0, 16)
    no_p = oracle.sweep(out["W2"], out["U"], None, 2, 0, 16)
    np.testing.assert_array_equal(out["codes"], with_p["codes"])
    assert np.any(no_p["codes"] != with_p["codes"])
    assert out["obj"] == pytest.approx(oracle.objective(out["W2"], with_p["what"], out["HX2"],
                                                        out["D2"], out["HG2"]), rel=1e-12)
    # the baseline rounds the same processed weights
    codes_rtn, what_rtn = oracle.rtn(out["W2"], 2)
    np.testing.assert_array_equal(out["codes_rtn"], codes_rtn)
    assert out["obj_rtn"] == pytest.approx(oracle.objective(out["W2"], what_rtn, out["HX2"],
                                                            out["D2"], out["HG2"]), rel=1e-12)


def test_grid_golden():
    for case in _load("grid.json")["cases"]:
        row = np.array([case["row"]], dtype=np.float32)
        sc, zr = oracle.grid_fp32(row, case["bits"])
        want_scale = case.get("scale", None)
        if want_scale is None:
            want_scale = np.float32(case["scale_num"]) / np.float32(case["scale_den"])
        assert sc[0] == np.float32(want_scale), case["why"]
        assert zr[0] == case["zero"], case["why"]
        codes, what = oracle.rtn(row, case["bits"])
        np.testing.assert_array_equal(codes[0], case["codes"], err_msg=case["why"])
        np.testing.assert_allclose(what[0], case["dequant"], atol=1e-7, err_msg=case["why"])


def test_group_grid_golden():
    """Group grids are taken from the working values when the sweep reaches
    the group (reading R6), feedback and drift term included; the hand-worked
    cases differ from grids taken from the original weights."""
    for case in _load("group_grid.json")["cases"]:
        W0 = np.array(case["W0"], dtype=np.float64)
        U = np.array(case["U"], dtype=np.float64)
        P = None if case["P"] is None else np.array(case["P"], dtype=np.float64)
        for block in (2, 4):  # lazy and unblocked forms agree
            res = oracle.sweep(W0, U, P, case["bits"], case["group"], block=block)
            np.testing.assert_array_equal(res["scale"], np.float32(case["scale"]), err_msg=case["name"])
            np.testing.assert_array_equal(res["zero"], np.float32(case["zero"]), err_msg=case["name"])
            np.testing.assert_array_equal(res["codes"], case["codes"], err_msg=case["name"])
            np.testing.assert_array_equal(res["what"], case["dequant"], err_msg=case["name"])
        other = np.float32(case["grid_from_W0_would_be"]["scale"])
        assert np.any(other != np.float32(case["scale"]))


def test_cv_in_out_golden():
    """CV_in runs over the input channels (columns), CV_out over the rows (reading R9)."""
    for case in _load("cv_in_out.json")["cases"]:
        cvi, cvo = oracle.cv_in_out(np.array(case["W"]))
        assert cvi * cvi == pytest.approx(case["cv_in_squared"], rel=1e-12, abs=1e-15), case["why"]
        assert cvo * cvo == pytest.approx(case["cv_out_squared"], rel=1e-12, abs=1e-15), case["why"]


def test_config0_objective_beats_rtn():
    spec = layer_specs(0)[0]
    L = make_layer(spec)
    out = oracle.quantize_layer(L["x"], L["xq"], L["g"], L["W"], L["sign_in"], L["sign_out"],
                                spec.bits, spec.group, spec.block, spec.damp)
    assert out["obj"] > 0 and out["obj"] < out["obj_rtn"]


# ------------------------------------------------------------------ allocation


def test_allocation_golden():
    for name in ("allocation.json", "allocation_ties.json"):
        a = _load(name)
        got = oracle.allocate_bits(a["s"], a["n_params"], a["widths"], a["avg_budget"])
        assert got == a["bits"], a["why"]


def _brute_force_alloc(s, n, widths, avg):
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    budget = avg * sum(n)
    best = None
    for bits in itertools.product(sorted(widths), repeat=len(s)):
        if sum(b * k for b, k in zip(bits, n)) > budget:
            continue
        key = tuple(bits[i] for i in order)
        if best is None or key > best[0]:
            best = (key, list(bits))
    return best[1]


def test_allocation_matches_brute_force():
    rng = np.random.default_rng(15)
    spec_n = [sp.n_params for sp in layer_specs(4)]
    for trial in range(40):
        s = list(rng.lognormal(0, 2, 7))
        if trial % 5 == 0:
            s[2] = s[1]  # ties resolved by input order
        n = spec_n if trial % 2 == 0 else list(rng.integers(1, 50, 7))
        avg = [2.5, 2.2, 3.0, 3.7][trial % 4]
        assert oracle.allocate_bits(s, n, (2, 3, 4), avg) == _brute_force_alloc(s, n, (2, 3, 4), avg)


@pytest.mark.parametrize("bits,block", [(2, 128), (3, 64), (4, 256)])
def test_folded_sweep_equals_literal_recursion(bits, block):
    """With one grid per channel (taken from W0), the sweep with the literal
    drift term W0_p P_{p, >p} added after each column equals the plain GPTQ
    sweep (P = 0) of the folded matrix W0 + W0 P: P is strictly upper and W0
    is constant, so the added terms sum to W0 P before any column is reached."""
    rng = np.random.default_rng(bits * 100 + block)
    n_tok, d_in, d_out = 600, 256, 24
    x = rng.standard_normal((n_tok, d_in)) * np.exp(rng.standard_normal(d_in))
    xq = x + 0.05 * rng.standard_normal((n_tok, d_in))
    HX, D, _ = oracle.covariances(x.astype(np.float32), xq.astype(np.float32), None)
    U = oracle.inv_factor(HX, 0.01)
    P = oracle.form_p(D, U)
    assert np.all(np.tril(P) == 0)
    W0 = 0.02 * rng.standard_normal((d_out, d_in))
    g = oracle.grid_fp32(W0.astype(np.float32), bits)
    lit = oracle.sweep(W0, U, P, bits, 0, block, grid0=g)
    fold = oracle.sweep(W0 + W0 @ P, U, None, bits, 0, block, grid0=g)
    np.testing.assert_array_equal(lit["codes"], fold["codes"])
    np.testing.assert_allclose(lit["what"], fold["what"], rtol=0, atol=1e-12)
