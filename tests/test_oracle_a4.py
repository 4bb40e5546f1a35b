"""Pins of the weight-and-activation reference (oracle/deploy.py:
quantize_activations, infer_a4) against a hand-worked vector, brute force
over the levels, exact scale invariance, inputs already on the 4-bit grid
(where it must reduce to the pinned weight-only product) and the dense
de-transformed matrix applied to the dequantized activation."""
import numpy as np
import pytest

import oracle
from oracle import deploy
from oracle.kronq import apply_hadamard_left


def test_quantize_hand_worked():
    # max |x| = 3.5 -> s = 3.5 / 7 = 0.5, t = x / s; rint ties go to even
    x = np.array([[1.75, -3.5, 0.875, 0.25, 0.125, 3.5, -1.25, 0.0]])
    r = deploy.quantize_activations(x, 4, 1.0)
    assert r["s"][0] == np.float32(0.5)
    assert list(r["q"][0]) == [4, -7, 2, 0, 0, 7, -2, 0]
    # clip 0.5 -> s = 0.25: values past the clip saturate, -14 at -8 and 14 at 7
    r = deploy.quantize_activations(x, 4, 0.5)
    assert r["s"][0] == np.float32(0.25)
    assert list(r["q"][0]) == [7, -8, 4, 1, 0, 7, -5, 0]
    # 3 bits: levels -4 .. 3, s = 3.5 / 3
    r = deploy.quantize_activations(np.array([[3.5, -3.5, 0.0]]), 3, 1.0)
    assert list(r["q"][0]) == [3, -3, 0]


def test_quantize_divides_in_fp32():
    """The rounded value is the fp32 quotient x2 / s, not x2 times the fp32
    reciprocal of s. With max |x| = 0.1875, s = fl(0.1875 / 7) and
    x = fl(1.5 s): the quotient is exactly 1.5, which rounds to 2 (ties to
    even), while x * fl(1 / s) = 1.4999999 would round to 1."""
    f = np.float32
    s = f(0.1875) / f(7)
    x = f(1.5) * s
    assert x / s == f(1.5) and x * (f(1) / s) < f(1.5)
    r = deploy.quantize_activations(np.array([[float(x), 0.1875]]), 4, 1.0)
    assert r["s"][0] == s and r["t"][0, 0] == f(1.5)
    assert list(r["q"][0]) == [2, 7]


@pytest.mark.parametrize("bits,clip", [(4, 1.0), (4, 0.9), (4, 0.6), (3, 1.0), (8, 0.8)])
def test_quantize_is_the_nearest_level(bits, clip):
    """Each code is the level nearest to x2 / s (brute force over all levels)."""
    rng = np.random.default_rng(bits * 10 + int(10 * clip))
    x = rng.standard_normal((6, 40)) * rng.uniform(1e-3, 1e3, (6, 1))
    r = deploy.quantize_activations(x, bits, clip)
    levels = np.arange(-(1 << (bits - 1)), 1 << (bits - 1))
    for b in range(6):
        t = r["t"][b].astype(np.float64)
        best = levels[np.argmin(np.abs(t[:, None] - levels[None, :]), axis=1)]
        np.testing.assert_array_equal(r["q"][b], best)
        if clip == 1.0:  # nothing saturates: every value within half a step
            xs = x[b].astype(np.float32).astype(np.float64)
            assert np.max(np.abs(xs - r["s"][b] * r["q"][b])) <= 0.5 * r["s"][b] * (1 + 1e-6)
            assert np.max(np.abs(r["q"][b])) == (1 << (bits - 1)) - 1


def test_quantize_scale_invariance_and_zero_vector():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 64))
    r0 = deploy.quantize_activations(x, 4, 0.9)
    for k in (-20, -3, 5, 30):
        r = deploy.quantize_activations(x * 2.0 ** k, 4, 0.9)
        np.testing.assert_array_equal(r["q"], r0["q"])
        np.testing.assert_array_equal(r["s"], r0["s"] * np.float32(2.0 ** k))
    r = deploy.quantize_activations(np.zeros((2, 16)), 4, 1.0)
    assert not r["q"].any() and not r["s"].any()


def _layer(d_out=64, d_in=128, blk_in=32, seed=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((300, d_in)) * np.exp(rng.standard_normal(d_in))
    g = rng.standard_normal((300, d_out)) * np.exp(rng.standard_normal(d_out))
    HX, _, HG = oracle.covariances(None, x.astype(np.float32), g.astype(np.float32))
    W = 0.02 * rng.standard_normal((d_out, d_in))
    si = rng.choice([-1, 1], d_in).astype(np.int8)
    so = rng.choice([-1, 1], d_out).astype(np.int8)
    _, _, _, _, s_x, s_g = oracle.biip(W, HX, None, HG, si, so, blk_in, 0)
    codes = rng.integers(0, 4, (d_out, d_in)).astype(np.uint8)
    scale = rng.uniform(0.01, 0.02, d_out).astype(np.float32)
    zero = rng.integers(0, 4, d_out).astype(np.float32)
    return dict(codes=codes, packed=deploy.pack_codes(codes, 2), scale=scale, zero=zero,
                s_x=s_x, s_g=s_g, si=si, so=so, rng=rng)


def _unrotate(x2, s_x, si, b):
    """x = S_X V^T x2 with V^T = diag(sign) blockdiag(H_b / sqrt b)."""
    return (np.asarray(si, np.float64)[:, None]
            * apply_hadamard_left(np.asarray(x2, np.float64).T, np.ones(x2.shape[1]), b)).T \
        * np.asarray(s_x, np.float64)[None, :]


def test_input_on_the_grid_reduces_to_weight_only():
    """x chosen so that V S_X^-1 x is an integer vector with largest magnitude
    7: the codes are that vector, s = 1, and the result is the weight-only
    product (deploy.infer, pinned to BiIP) of the same x."""
    L = _layer()
    k = L["rng"].integers(-7, 8, (3, 128)).astype(np.float64)
    k[:, 5] = [7, -7, 7]
    x = _unrotate(k, L["s_x"], L["si"], 32)
    r = deploy.infer_a4(x, L["packed"], 2, L["scale"], L["zero"], 0, L["s_x"], L["s_g"],
                        L["si"], L["so"], 32, 0)
    np.testing.assert_array_equal(r["q"], k.astype(np.int8))
    np.testing.assert_array_equal(r["s"], np.ones(3, np.float32))
    y = deploy.infer(x, L["packed"], 2, L["scale"], L["zero"], 0, L["s_x"], L["s_g"], L["si"], L["so"], 32, 0)
    np.testing.assert_allclose(r["y"], y, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("clip", [1.0, 0.85])
def test_infer_a4_is_the_dense_layer_on_the_dequantized_input(clip):
    """y = W^ x^ with W^ the de-transformed dequantized layer and x^ = S_X V^T
    (s q) the dequantized activation taken back to the original basis."""
    L = _layer(seed=7)
    x = L["rng"].standard_normal((4, 128)) * 3.0
    r = deploy.infer_a4(x, L["packed"], 2, L["scale"], L["zero"], 0, L["s_x"], L["s_g"],
                        L["si"], L["so"], 32, 0, clip=clip)
    dense = deploy.detransform(deploy.dequantize(L["codes"], L["scale"], L["zero"]), L["s_x"], L["s_g"],
                               L["si"], L["so"], 32, 0)
    xhat = _unrotate(r["s"].astype(np.float64)[:, None] * r["q"], L["s_x"], L["si"], 32)
    np.testing.assert_allclose(r["y"], xhat @ dense.T, rtol=1e-10, atol=1e-12)
    # and x^ is close to x: the activation error is at most half a step per
    # rotated value when nothing saturates
    if clip == 1.0:
        x2 = deploy.rotate_input(x, L["s_x"], L["si"], 32)
        err = np.abs(x2 - r["s"].astype(np.float64)[:, None] * r["q"])
        assert np.all(err <= 0.5 * r["s"][:, None] * (1 + 1e-6))
