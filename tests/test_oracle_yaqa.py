"""Pins of oracle/yaqa.py (rounding with output-side feedback) against what
the pages and the mathematics fix, not against the oracle's own formulas:

* the pages' literal fixed-point iteration (notes on YAQA, key design 4,
  Eq. 5/6, built from the LDL factors of H) reaches the row-major oracle's
  codes within the m + n - 1 steps of key design 1;
* the LDL factor reproduces H and the library-Cholesky inverse factor;
* the rounding residuals decouple the Kronecker objective exactly;
* with H_O = I the rounding is the (already pinned) GPTQ / GPTAQ sweep, and
  with H_O = H_I = I it is round-to-nearest;
* transposing W swaps the roles of the two factors.
"""
import numpy as np
import pytest

from oracle import kronq, yaqa


def _cov(d, n_tok, rng, outliers=2):
    """E[x x^T] of lognormal-scaled channels with a few x20 outliers, like the
    layer workloads (fp64)."""
    s = rng.lognormal(0.0, 1.0, d)
    s[:outliers] *= 20.0
    X = rng.standard_normal((n_tok, d)) * s
    return X.T @ X / n_tok


def _layer(m, n, rng, bits):
    W0 = rng.normal(0.0, 0.02, (m, n))
    HI = kronq.damped(_cov(n, 4 * n, rng), 0.01)
    HO = kronq.damped(_cov(m, 4 * m, rng), 0.01)
    UI = kronq.inv_factor(HI, 0.0)
    UO = kronq.inv_factor(HO, 0.0)
    sc, zr = kronq.grid_fp32(W0.astype(np.float32), bits)
    return W0, HI, HO, UI, UO, sc, zr


def test_ldl_upper_definition():
    rng = np.random.default_rng(5)
    H = kronq.damped(_cov(37, 200, rng), 0.01)
    A, d = yaqa.ldl_upper(H)
    assert np.all(d > 0)
    np.testing.assert_array_equal(np.tril(A, -1), 0.0)
    np.testing.assert_allclose(np.diag(A), 1.0, rtol=0, atol=0)
    np.testing.assert_allclose(A @ np.diag(d) @ A.T, H, rtol=1e-11, atol=1e-11 * np.abs(H).max())
    # U^T U = H^-1 with U upper: the factor is D^-1/2 A^-1 (another route:
    # invert, then library Cholesky)
    U = kronq.inv_factor(H, 0.0)
    np.testing.assert_allclose(np.diag(d ** -0.5) @ np.linalg.inv(A), U, rtol=1e-8,
                               atol=1e-9 * np.abs(U).max())


@pytest.mark.parametrize("m,n,bits,seed", [(12, 20, 2, 0), (20, 12, 3, 1), (16, 16, 4, 2),
                                           (9, 31, 2, 3), (24, 40, 3, 4)])
def test_fixed_point_of_the_pages_equals_row_major(m, n, bits, seed):
    rng = np.random.default_rng(100 + seed)
    W0, HI, HO, UI, UO, sc, zr = _layer(m, n, rng, bits)
    fp_codes, fp_what, changed = yaqa.fixed_point(W0, HI, HO, sc, zr, bits)
    assert not changed, "not a fixed point after m + n - 1 iterations"
    res = yaqa.round_two_sided(W0, UI, UO, sc, zr, bits)
    np.testing.assert_array_equal(res["codes"], fp_codes)
    np.testing.assert_allclose(res["what"], fp_what, rtol=0, atol=1e-12)
    # the feedback matters: plain rounding gives other codes
    rtn_codes, _ = kronq.rtn(W0, bits)
    assert np.any(rtn_codes != fp_codes)


def test_fixed_point_settles_by_antidiagonals():
    """The nilpotency argument of key design 1: entry (i, j) is fed back only
    from entries above-left of it, so after k iterations every entry with
    i + j <= k holds its final code, whatever the rest still does."""
    rng = np.random.default_rng(300)
    m, n, bits = 10, 13, 2
    W0, HI, HO, UI, UO, sc, zr = _layer(m, n, rng, bits)
    full, _, changed = yaqa.fixed_point(W0, HI, HO, sc, zr, bits)
    assert not changed
    ii, jj = np.indices((m, n))
    for k in (0, 1, 4, 9, 15):
        part, _, _ = yaqa.fixed_point(W0, HI, HO, sc, zr, bits, iters=k)
        done = ii + jj <= k
        np.testing.assert_array_equal(part[done], full[done])


def test_fixed_point_default_covers_the_longest_chain():
    """A 3 x 4 case whose codes settle only after m + n - 2 = 5 iterations
    (the longest above-left chain of a 3 x 4 array, key design 1): the
    default count reaches the row-major result, one iteration fewer does not,
    so a count tied to max(m, n) alone would stop too early. Found by a
    search over seeds of this recipe (well-conditioned random factors,
    condition number up to 1e3, N(0, 1) weights, 3 bits)."""
    rng = np.random.default_rng(50)
    m, n, bits = 3, 4, 3

    def spd(k):
        q, _ = np.linalg.qr(rng.standard_normal((k, k)))
        return (q * np.exp(rng.uniform(0, np.log(1e3), k))) @ q.T

    HI, HO = spd(n), spd(m)
    W0 = rng.standard_normal((m, n))
    sc, zr = kronq.grid_fp32(W0.astype(np.float32), bits)
    ref = yaqa.round_two_sided(W0, kronq.inv_factor(HI, 0.0), kronq.inv_factor(HO, 0.0), sc, zr, bits)
    codes, _, changed = yaqa.fixed_point(W0, HI, HO, sc, zr, bits)
    assert not changed
    np.testing.assert_array_equal(codes, ref["codes"])
    early, _, changed = yaqa.fixed_point(W0, HI, HO, sc, zr, bits, iters=m + n - 3)
    assert changed or np.any(early != ref["codes"])


def test_forced_replay_midpoint_distance_hand_worked():
    """Row [-0.25, 0.5] on the grid scale 0.25, zero 1 (2 bits), no feedback:
    entry 0 has w/scale = -1 -> code 0; forced to 1 the midpoint of codes 0
    and 1 lies at 0.5 - 1 = -0.5 grid steps, a distance of 0.5; entry 1 is
    0.5/0.25 = 2 -> code 3."""
    res = yaqa.round_two_sided(np.array([[-0.25, 0.5]]), np.eye(2), np.eye(1), np.float32(0.25),
                               np.float32(1.0), 2, forced_codes=np.array([[1, 3]]))
    assert res["mismatches"] == [(0, 0, 0, 1, 0.5)]
    np.testing.assert_array_equal(res["codes"], [[1, 3]])
    np.testing.assert_array_equal(res["what"], [[0.0, 0.5]])


@pytest.mark.parametrize("m,n,bits", [(16, 24, 2), (24, 16, 4)])
def test_residuals_decouple_the_kronecker_objective(m, n, bits):
    """tr(Delta H_I Delta^T H_O) = sum_ij eps_ij^2 d_O,i d_I,j with
    Delta = W* - W^ and eps the rounding residuals: the identity that makes
    the triangular feedback the right one (reading R-Y1)."""
    rng = np.random.default_rng(7 * m + n)
    W0, HI, HO, UI, UO, sc, zr = _layer(m, n, rng, bits)
    res = yaqa.round_two_sided(W0, UI, UO, sc, zr, bits)
    lhs = yaqa.kron_objective(W0 - res["what"], HI, HO)
    dI = yaqa.ldl_upper(HI)[1]
    dO = yaqa.ldl_upper(HO)[1]
    rhs = float(np.sum(res["eps"] ** 2 * dO[:, None] * dI[None, :]))
    assert abs(lhs - rhs) <= 1e-9 * rhs


@pytest.mark.parametrize("with_p", [False, True])
def test_identity_output_factor_is_the_kronq_sweep(with_p):
    rng = np.random.default_rng(11 + with_p)
    m, n, bits = 24, 256, 2
    W0, HI, HO, UI, UO, sc, zr = _layer(m, n, rng, bits)
    P = None
    if with_p:
        Xq = rng.standard_normal((4 * n, n))
        D = (1e-2 * rng.standard_normal((4 * n, n))).T @ Xq / (4 * n)
        P = kronq.form_p(D, UI)
    res = yaqa.quantize_two_sided(W0, UI, np.eye(m), bits, P=P)
    ref = kronq.sweep(W0, UI, P, bits, 0, 128)
    np.testing.assert_array_equal(res["codes"], ref["codes"])
    np.testing.assert_allclose(res["what"], ref["what"], rtol=0, atol=1e-12)


def test_identity_factors_are_round_to_nearest():
    rng = np.random.default_rng(17)
    W0 = rng.normal(0.0, 0.02, (10, 33))
    res = yaqa.quantize_two_sided(W0, np.eye(33), np.eye(10), 3)
    np.testing.assert_array_equal(res["codes"], kronq.rtn(W0, 3)[0])


def test_transpose_swaps_the_factors():
    rng = np.random.default_rng(23)
    m, n, bits = 14, 22, 2
    W0, HI, HO, UI, UO, _, _ = _layer(m, n, rng, bits)
    sc, zr = np.float32(0.02), np.float32(2.0)  # one grid for every entry
    a = yaqa.round_two_sided(W0, UI, UO, sc, zr, bits)
    b = yaqa.round_two_sided(W0.T, UO, UI, sc, zr, bits)
    np.testing.assert_array_equal(a["codes"], b["codes"].T)


def test_output_feedback_lowers_the_kronecker_objective():
    """The point of the output-side term: on the Kronecker objective the
    two-sided rounding beats the one-sided (GPTQ) rounding of the same target
    on average over seeds."""
    two, one = [], []
    for seed in range(4):
        rng = np.random.default_rng(500 + seed)
        m, n, bits = 32, 48, 2
        W0, HI, HO, UI, UO, sc, zr = _layer(m, n, rng, bits)
        a = yaqa.round_two_sided(W0, UI, UO, sc, zr, bits)
        b = yaqa.round_two_sided(W0, UI, np.eye(m), sc, zr, bits)
        two.append(yaqa.kron_objective(W0 - a["what"], HI, HO))
        one.append(yaqa.kron_objective(W0 - b["what"], HI, HO))
    assert np.mean(two) < np.mean(one)


@pytest.mark.parametrize("with_p", [False, True])
def test_residuals_recovered_from_the_result(with_p):
    """The any-size check: the residuals solved back from (W*, W^) are the
    ones the rounding produced, and they lie within half a grid step; a
    result rounded with the output feedback left out fails the check."""
    rng = np.random.default_rng(41 + with_p)
    m, n, bits = 20, 36, 2
    W0, HI, HO, UI, UO, sc, zr = _layer(m, n, rng, bits)
    P = None
    Wt = W0
    if with_p:
        D = 1e-3 * rng.standard_normal((n, n))
        P = kronq.form_p(D, UI)
        Wt = W0 + W0 @ P
    res = yaqa.quantize_two_sided(W0, UI, UO, bits, P=P)
    eps = yaqa.residuals_of(Wt, res["what"], UI, UO)
    np.testing.assert_allclose(eps, res["eps"], rtol=0, atol=1e-10)
    assert yaqa.rounding_violation(eps, res["codes"], res["scale"], bits) <= 1e-9
    one = yaqa.quantize_two_sided(W0, UI, np.eye(m), bits, P=P)
    eps1 = yaqa.residuals_of(Wt, one["what"], UI, UO)
    assert yaqa.rounding_violation(eps1, one["codes"], one["scale"], bits) > 0.05
