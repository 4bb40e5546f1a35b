"""GPU parity of the solver with the 128- and 256-wide fp32 product tiles,
and the three-term bf16 product kernel, forced.

The library chooses the product kernel by shape, and the small shapes of the
other parity tests all take the 64-wide fp32 tile. Here kq_set_gemm_tile(128)
and kq_set_gemm_tile(256) force the large-tile kernel, and
kq_set_gemm_tile(3) the kernel that runs fp32 products as six products of
three-term bf16 splits on the bf16 matrix cores, into every product that
allows it, at sizes that are not multiples of the tile (ragged tiles in M,
N and K), with triangular
operands (factorization updates, triangular inverse, P, the fold), batched
products (inverse levels) and triangular outputs, and the results are held
to the same bars as the default path: the inverse factor by its backward
error, P to 1e-5 relative, codes by forced replay of the oracle, the layer
objective to 1e-4 relative.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import code_report, dev, have_gpu, host, rel_fro, spd

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

if have_gpu():
    import post_weight_quantization_amd as kq


@pytest.fixture(autouse=True, params=[128, 256, 3])
def large_tiles(request):
    kq.kq_set_gemm_tile(request.param)
    yield request.param
    kq.kq_set_gemm_tile(0)


@pytest.mark.parametrize("n,cond", [(256, 1e3), (384, 1e3), (640, 1e4), (1152, 1e3)])
def test_cholesky_inv_backward_error_large_tiles(n, cond):
    rng = np.random.default_rng(n + 1)
    H = spd(rng, n, cond).astype(np.float32)
    U = host(kq.kq_cholesky_inv(dev(H), 0.01)).astype(np.float64)
    assert np.all(np.tril(U, -1) == 0)
    Hd = oracle.damped(H.astype(np.float64), 0.01)
    kappa = np.linalg.cond(Hd)
    resid = np.linalg.norm(U.T @ U @ Hd - np.eye(n)) / np.sqrt(n)
    fwd = rel_fro(U, oracle.inv_factor(H, 0.01))
    print(f"n={n} cond(Hd)={kappa:.3g} resid={resid:.3g} fwd={fwd:.3g}")
    assert resid < 1e-6 * kappa
    assert fwd < 1e-6 * kappa


@pytest.mark.parametrize("n", [384, 640])
def test_form_p_large_tiles(n):
    rng = np.random.default_rng(n + 2)
    H = spd(rng, n, 1e3)
    U = oracle.inv_factor(H, 0.01).astype(np.float32)
    D = (0.05 * rng.standard_normal((n, n))).astype(np.float32)
    P = host(kq.kq_form_p(dev(D), dev(U)))
    assert np.all(np.tril(P) == 0)
    assert rel_fro(P, oracle.form_p(D, U)) < 1e-5


@pytest.mark.parametrize("d_out,n,bits,group", [(200, 512, 2, 0), (300, 384, 3, 128), (257, 640, 4, 0)])
def test_gptaq_forced_replay_large_tiles(d_out, n, bits, group):
    rng = np.random.default_rng(d_out * n)
    H = spd(rng, n, 1e3)
    U = oracle.inv_factor(H, 0.01).astype(np.float32)
    D = (0.02 * rng.standard_normal((n, n))).astype(np.float32)
    W0 = (0.02 * rng.standard_normal((d_out, n))).astype(np.float32)
    tW = dev(W0)
    codes, scale, zero = kq.kq_gptaq_quantize(tW, dev(U), dev(D), bits, group)
    codes, scale, zero, What = host(codes), host(scale), host(zero), host(tW)
    P = oracle.form_p(D, U)
    ref = oracle.sweep(W0, U, P, bits, group, 128, forced_codes=codes,
                       forced_grid=(scale, zero) if group else None)
    rep = code_report(ref, codes.size)
    assert rep["n"] <= max(1, int(1e-4 * codes.size)), rep
    assert rep["worst"] <= 1e-4, rep
    np.testing.assert_allclose(What, ref["what"], rtol=1e-5, atol=1e-6)


def test_layer_objective_large_tiles():
    rng = np.random.default_rng(12)
    d_out, n = 300, 384
    HX = spd(rng, n, 1e3).astype(np.float32)
    HG = spd(rng, d_out, 1e3).astype(np.float32)
    D = (0.01 * rng.standard_normal((n, n))).astype(np.float32)
    W0 = (0.02 * rng.standard_normal((d_out, n))).astype(np.float32)
    Wh = (W0 + 0.002 * rng.standard_normal((d_out, n))).astype(np.float32)
    got = kq.kq_layer_objective(dev(W0), dev(Wh), dev(HX), dev(D), dev(HG))
    assert got == pytest.approx(oracle.objective(W0, Wh, HX, D, HG), rel=1e-4)


def test_tiles_agree(large_tiles):
    """The same factorization on the forced kernel and the 64-wide tile:
    fp32 results that differ only in rounding and summation order."""
    rng = np.random.default_rng(5)
    n = 640
    H = dev(spd(rng, n, 1e3).astype(np.float32))
    U_large = host(kq.kq_cholesky_inv(H, 0.01)).astype(np.float64)
    kq.kq_set_gemm_tile(64)
    U64 = host(kq.kq_cholesky_inv(H, 0.01)).astype(np.float64)
    assert rel_fro(U_large, U64) < 1e-5
