"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (from the quantization target): covariances <= 1e-4 relative
Frobenius; sensitivity <= 1e-5 relative; layer objective <= 1e-3 relative;
integer codes identical on >= 99.99% of entries with every mismatch at a
pre-rounding value within 1e-4 of a grid step from the rounding midpoint
(checked by forced replay of the oracle on the GPU's own stage inputs, so one
legitimate flip does not cascade along a row). Stage outputs in fp32 whose
error is pure rounding (BiIP, P) are held to 1e-5; the inverse factor is held
by its backward error.
"""
import numpy as np
import pytest

import oracle
from synth import layer_specs, make_layer
from tests.gpu_util import code_report, dev, have_gpu, host, rel_fro, spd, tile_rel_fro

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

if have_gpu():
    import torch

    import post_weight_quantization_amd as kq
    from post_weight_quantization_amd import _native as N


def _bf16(rng, shape, scale=1.0):
    from synth import f32_to_bf16_bits
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


# ------------------------------------------------------------------ stage 1


def test_cov_f32_config0():
    spec = layer_specs(0)[0]
    L = make_layer(spec)
    HX, D, HG = kq.kq_accumulate_cov(dev(L["x"]), dev(L["xq"]), dev(L["g"]), 1.0 / spec.n_tok, 0.0)
    oHX, oD, oHG = oracle.covariances(L["x"], L["xq"], L["g"])
    assert rel_fro(host(HX), oHX) < 1e-5
    assert rel_fro(host(D), oD) < 1e-5
    assert rel_fro(host(HG), oHG) < 1e-5
    # tile by tile too: the outlier channels dominate the whole-matrix norm
    for got, ref in ((HX, oHX), (D, oD), (HG, oHG)):
        assert tile_rel_fro(host(got), ref, 64) < 1e-4


# ragged tiles and token tails; one token; a tail only (no full 32-token
# stage); one full stage plus one token; the minimum width of 8 channels
@pytest.mark.parametrize("n_tok,d_in,d_out", [(1000, 264, 512), (4096, 512, 256), (64, 256, 8),
                                              (1, 8, 8), (31, 264, 24), (33, 8, 520)])
def test_cov_bf16_ragged(n_tok, d_in, d_out):
    rng = np.random.default_rng(n_tok + d_in)
    sig = np.exp(rng.standard_normal(d_in)).astype(np.float32)
    x32 = (rng.standard_normal((n_tok, d_in)) * sig).astype(np.float32)
    from synth import f32_to_bf16_bits
    X = f32_to_bf16_bits(x32)
    Xq = f32_to_bf16_bits(x32 + (0.01 * sig * rng.standard_normal((n_tok, d_in))).astype(np.float32))
    G = _bf16(rng, (n_tok, d_out), 3.0)
    HX, D, HG = kq.kq_accumulate_cov(dev(X), dev(Xq), dev(G), 1.0 / n_tok, 0.0)
    torch.cuda.synchronize()
    oHX, oD, oHG = oracle.covariances(X, Xq, G)
    assert rel_fro(host(HX), oHX) < 1e-4
    assert rel_fro(host(D), oD) < 1e-4
    assert rel_fro(host(HG), oHG) < 1e-4
    for got, ref in ((HX, oHX), (D, oD), (HG, oHG)):
        assert tile_rel_fro(host(got), ref, 64) < 1e-4
    # symmetric outputs are exactly mirrored
    np.testing.assert_array_equal(host(HX), host(HX).T)
    np.testing.assert_array_equal(host(HG), host(HG).T)


@pytest.mark.parametrize("want", [("HX",), ("D",), ("HG",), ("HX", "HG"), ("D", "HG")])
def test_cov_bf16_output_subsets(want):
    """Any subset of the three outputs may be requested (the others are NULL
    and skipped); each requested one matches the oracle."""
    rng = np.random.default_rng(len(want) * 7 + len(want[0]))
    n_tok, d_in, d_out = 700, 264, 136
    X = _bf16(rng, (n_tok, d_in), 1.0)
    Xq = _bf16(rng, (n_tok, d_in), 1.0)
    G = _bf16(rng, (n_tok, d_out), 2.0)
    HX, D, HG = kq.kq_accumulate_cov(dev(X), dev(Xq), dev(G), 1.0 / n_tok, 0.0, want=want)
    oHX, oD, oHG = oracle.covariances(X, Xq, G)
    for name, got, ref in (("HX", HX, oHX), ("D", D, oD), ("HG", HG, oHG)):
        if name in want:
            assert rel_fro(host(got), ref) < 1e-4, name
            assert tile_rel_fro(host(got), ref, 64) < 1e-4, name
        else:
            assert got is None, name


def test_cov_bf16_chunked_beta():
    rng = np.random.default_rng(3)
    n, d_in, d_out = 3000, 256, 256
    X = _bf16(rng, (n, d_in))
    Xq = _bf16(rng, (n, d_in))
    G = _bf16(rng, (n, d_out))
    tX, tXq, tG = dev(X), dev(Xq), dev(G)
    HX, D, HG = kq.kq_accumulate_cov(tX[:1200].contiguous(), tXq[:1200].contiguous(),
                                     tG[:1200].contiguous(), 1.0 / n, 0.0)
    kq.kq_accumulate_cov(tX[1200:].contiguous(), tXq[1200:].contiguous(), tG[1200:].contiguous(),
                         1.0 / n, 1.0, HX=HX, D=D, HG=HG)
    oHX, oD, oHG = oracle.covariances(X, Xq, G)
    assert rel_fro(host(HX), oHX) < 1e-4
    assert rel_fro(host(D), oD) < 1e-4
    assert rel_fro(host(HG), oHG) < 1e-4
    for got, ref in ((HX, oHX), (D, oD), (HG, oHG)):
        assert tile_rel_fro(host(got), ref, 64) < 1e-4


# ------------------------------------------------------------------ stage 2


def _spd_large(rng, n, k=96):
    """A cheap SPD matrix for large n: low-rank Gram matrix plus a spread diagonal."""
    Z = rng.standard_normal((n, k))
    return Z @ Z.T / k + np.diag(np.exp(rng.uniform(0, np.log(1e3), n)))


# (4096, 4096) and (8192, 4096): the workloads' Hadamard blocks of 4096 and
# 8192 on both sides (compile-time row passes, two column passes)
@pytest.mark.parametrize("d_out,d_in,bo,bi", [(256, 256, 0, 0), (384, 512, 128, 0), (1024, 4096, 0, 64),
                                              (4096, 4096, 0, 0), (8192, 4096, 0, 0)])
def test_biip_against_oracle(d_out, d_in, bo, bi):
    rng = np.random.default_rng(d_out + d_in)
    sc = np.exp(rng.standard_normal(d_in))
    big = max(d_out, d_in) > 2048
    HX = (_spd_large(rng, d_in) if big else spd(rng, d_in, 1e3)) * np.outer(sc, sc)  # diagonals over decades
    HG = _spd_large(rng, d_out) if big else spd(rng, d_out, 1e4)
    D = 0.01 * rng.standard_normal((d_in, d_in))
    W = 0.02 * rng.standard_normal((d_out, d_in))
    si = rng.choice([-1, 1], d_in).astype(np.int8)
    so = rng.choice([-1, 1], d_out).astype(np.int8)
    f32 = lambda a: np.asarray(a, np.float32)
    tW, tHX, tD, tHG = dev(f32(W)), dev(f32(HX)), dev(f32(D)), dev(f32(HG))
    s_x, s_g = kq.kq_biip(tW, tHX, tD, tHG, dev(si), dev(so), bi, bo)
    W2, HX2, D2, HG2, ox, og = oracle.biip(f32(W), f32(HX), f32(D), f32(HG), si, so, bi, bo)
    assert rel_fro(host(s_x), ox) < 1e-6
    assert rel_fro(host(s_g), og) < 1e-6
    assert rel_fro(host(tW), W2) < 1e-5
    assert rel_fro(host(tHX), HX2) < 1e-5
    assert rel_fro(host(tD), D2) < 1e-5
    assert rel_fro(host(tHG), HG2) < 1e-5
    # tile by tile: a wrong tile of small entries cannot hide behind the large ones
    for got, ref in ((tW, W2), (tHX, HX2), (tD, D2), (tHG, HG2)):
        assert tile_rel_fro(host(got), ref, 64) < 1e-4


@pytest.mark.parametrize("d_out,d_in,bo,bi", [(8, 8, 0, 0), (24, 40, 8, 8), (100, 36, 4, 4)])
def test_biip_small_and_degenerate(d_out, d_in, bo, bi):
    """Small shapes and blocks, with a zero column and a zero row in W and
    a zero diagonal entry of H_X and of H_G: their scales are 1 (reading R3)
    and everything else matches the oracle."""
    rng = np.random.default_rng(d_out * d_in)
    HX = spd(rng, d_in, 1e2)
    HX[2, :] = 0.0
    HX[:, 2] = 0.0
    HG = spd(rng, d_out, 1e2)
    HG[1, :] = 0.0
    HG[:, 1] = 0.0
    D = 0.01 * rng.standard_normal((d_in, d_in))
    W = 0.02 * rng.standard_normal((d_out, d_in))
    W[:, 5] = 0.0
    W[3, :] = 0.0
    si = rng.choice([-1, 1], d_in).astype(np.int8)
    so = rng.choice([-1, 1], d_out).astype(np.int8)
    f32 = lambda a: np.asarray(a, np.float32)
    tW, tHX, tD, tHG = dev(f32(W)), dev(f32(HX)), dev(f32(D)), dev(f32(HG))
    s_x, s_g = kq.kq_biip(tW, tHX, tD, tHG, dev(si), dev(so), bi, bo)
    W2, HX2, D2, HG2, ox, og = oracle.biip(f32(W), f32(HX), f32(D), f32(HG), si, so, bi, bo)
    sx, sg = host(s_x), host(s_g)
    assert sx[2] == 1.0 and sx[5] == 1.0 and sg[1] == 1.0 and sg[3] == 1.0
    assert rel_fro(sx, ox) < 1e-6
    assert rel_fro(sg, og) < 1e-6
    for got, ref in ((tW, W2), (tHX, HX2), (tD, D2), (tHG, HG2)):
        assert rel_fro(host(got), ref) < 1e-5
        assert tile_rel_fro(host(got), ref, 4) < 1e-4


# ------------------------------------------------------------------ stage 5


def test_sensitivity_exact_on_gpu_inputs():
    rng = np.random.default_rng(7)
    HX = spd(rng, 512).astype(np.float32)
    HG = spd(rng, 256).astype(np.float32)
    tx, tg, s = kq.kq_sensitivity(dev(HX), dev(HG))
    ox, og, os_ = oracle.sensitivity(HX, HG)
    assert tx == pytest.approx(ox, rel=1e-12)
    assert tg == pytest.approx(og, rel=1e-12)
    assert s == pytest.approx(os_, rel=1e-12)


# ------------------------------------------------------------------ stage 3


# 1664 and 2176: three and four 512-column superblocks and a ragged last one
# (trailing updates between superblocks, a narrow last superblock)
@pytest.mark.parametrize("n,cond", [(128, 1e2), (256, 1e3), (384, 1e3), (640, 1e4), (896, 1e3), (1024, 1e3),
                                    (1664, 1e3), (2176, 1e4)])
def test_cholesky_inv_backward_error(n, cond):
    rng = np.random.default_rng(n)
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


def test_cholesky_not_pd_reports_column():
    n = 256
    H = np.eye(n, dtype=np.float32)
    H[200, 200] = -1.0  # reversed order meets index 200 after 255..201
    with pytest.raises(kq.KQError) as ei:
        kq.kq_cholesky_inv(dev(H), 0.0)
    assert ei.value.status == N.KQ_ERR_NOT_PD
    assert ei.value.info == 201


# ------------------------------------------------------------------ stage 4


def test_form_p_against_oracle():
    rng = np.random.default_rng(9)
    n = 512
    H = spd(rng, n, 1e3)
    U = oracle.inv_factor(H, 0.01).astype(np.float32)
    D = (0.05 * rng.standard_normal((n, n))).astype(np.float32)
    P = host(kq.kq_form_p(dev(D), dev(U)))
    Po = oracle.form_p(D, U)
    assert np.all(np.tril(P) == 0)
    assert rel_fro(P, Po) < 1e-5


def _sweep_case(d_out, n, bits, group, with_d, seed):
    rng = np.random.default_rng(seed)
    H = spd(rng, n, 1e3)
    U = oracle.inv_factor(H, 0.01).astype(np.float32)
    D = (0.02 * rng.standard_normal((n, n))).astype(np.float32) if with_d else None
    W0 = (0.02 * rng.standard_normal((d_out, n))).astype(np.float32)
    tW = dev(W0)
    codes, scale, zero = kq.kq_gptaq_quantize(tW, dev(U), dev(D) if with_d else None, bits, group)
    codes, scale, zero, What = host(codes), host(scale), host(zero), host(tW)
    P = oracle.form_p(D, U) if with_d else None
    ref = oracle.sweep(W0, U, P, bits, group, 128, forced_codes=codes,
                       forced_grid=(scale, zero) if group else None)
    return W0, codes, scale, zero, What, ref


@pytest.mark.parametrize("d_out,n,bits,group,with_d", [
    (64, 256, 2, 0, False), (200, 512, 2, 0, True), (256, 384, 3, 128, True),
    (96, 256, 4, 128, False), (33, 128, 2, 0, True),
    (64, 256, 8, 0, True), (40, 128, 1, 0, False), (1, 256, 2, 128, True)])
def test_gptaq_forced_replay(d_out, n, bits, group, with_d):
    W0, codes, scale, zero, What, ref = _sweep_case(d_out, n, bits, group, with_d, d_out + n)
    rep = code_report(ref, codes.size)
    assert rep["n"] <= max(1, int(1e-4 * codes.size)), rep
    assert rep["worst"] <= 1e-4, rep
    if not group:
        # per-channel grid from the same fp32 W0: bit-exact
        sc, zr = oracle.grid_fp32(W0, bits)
        np.testing.assert_array_equal(scale[:, 0], sc)
        np.testing.assert_array_equal(zero[:, 0], zr)
    else:
        for smax, nz in ref["grid_mismatch"]:
            assert smax < 1e-5 and nz == 0
    # dequantized values follow the codes exactly
    sc = np.repeat(scale, group, axis=1) if group else scale
    zr = np.repeat(zero, group, axis=1) if group else zero
    np.testing.assert_allclose(What, sc * (codes.astype(np.float32) - zr), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(What, ref["what"], rtol=1e-5, atol=1e-6)


# -------------------------------------------------------------- objective


def test_layer_objective_against_oracle():
    rng = np.random.default_rng(11)
    d_out, n = 256, 512
    HX = spd(rng, n, 1e3).astype(np.float32)
    HG = spd(rng, d_out, 1e3).astype(np.float32)
    D = (0.01 * rng.standard_normal((n, n))).astype(np.float32)
    W0 = (0.02 * rng.standard_normal((d_out, n))).astype(np.float32)
    Wh = (W0 + 0.002 * rng.standard_normal((d_out, n))).astype(np.float32)
    got = kq.kq_layer_objective(dev(W0), dev(Wh), dev(HX), dev(D), dev(HG))
    want = oracle.objective(W0, Wh, HX, D, HG)
    assert got == pytest.approx(want, rel=1e-4)


# -------------------------------------------------------------- end to end


def test_config0_end_to_end():
    spec = layer_specs(0)[0]
    L = make_layer(spec)
    ref = oracle.quantize_layer(L["x"], L["xq"], L["g"], L["W"], L["sign_in"], L["sign_out"],
                                spec.bits, spec.group, spec.block, spec.damp)
    HX, D, HG = kq.kq_accumulate_cov(dev(L["x"]), dev(L["xq"]), dev(L["g"]), 1.0 / spec.n_tok, 0.0)
    assert rel_fro(host(HX), ref["HX"]) < 1e-4
    assert rel_fro(host(D), ref["D"]) < 1e-4
    assert rel_fro(host(HG), ref["HG"]) < 1e-4
    W = dev(L["W"])
    kq.kq_biip(W, HX, D, HG, dev(L["sign_in"]), dev(L["sign_out"]))
    W0p = host(W).copy()
    _, _, s = kq.kq_sensitivity(HX, HG)
    assert s == pytest.approx(ref["s"], rel=1e-5)
    U = kq.kq_cholesky_inv(HX, spec.damp)
    codes, scale, zero = kq.kq_gptaq_quantize(W, U, D, spec.bits, spec.group)
    obj = kq.kq_layer_objective(dev(W0p), W, HX, D, HG)
    assert obj == pytest.approx(ref["obj"], rel=1e-3)
    # codes: forced replay on the GPU's own stage inputs
    Uh, Dh = host(U), host(D)
    rep = oracle.sweep(W0p, Uh, oracle.form_p(Dh, Uh), spec.bits, spec.group, spec.block,
                       forced_codes=host(codes))
    r = code_report(rep, W0p.size)
    assert r["frac"] <= 1e-4 and r["worst"] <= 1e-4, r
    assert obj < ref["obj_rtn"]
