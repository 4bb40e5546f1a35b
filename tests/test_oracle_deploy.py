"""Pins of the inference reference (oracle/deploy.py) against hand-computed
packings, the forward BiIP transform it must undo, and the dense product."""
import numpy as np
import pytest

import oracle
from oracle import deploy


def test_packed_row_words():
    assert deploy.packed_row_words(4096, 2) == 256
    assert deploy.packed_row_words(4096, 3) == 384
    assert deploy.packed_row_words(33, 2) == 4    # 66 bits -> 3 words -> padded to 4
    assert deploy.packed_row_words(1, 4) == 4
    assert deploy.packed_row_words(11008, 3) == 1032


def test_pack_golden_words():
    # 2-bit codes 1, 2, 3, 0 -> bits 01 | 10 << 2 | 11 << 4 = 0b111001 = 57
    p = deploy.pack_codes(np.array([[1, 2, 3, 0]], np.uint8), 2)
    assert p.shape == (1, 4) and p[0, 0] == 57 and not p[0, 1:].any()
    # eleven 3-bit sevens fill bits 0..32: the 11th code straddles words 0 and 1
    p = deploy.pack_codes(np.full((1, 11), 7, np.uint8), 3)
    assert list(p[0]) == [0xFFFFFFFF, 0x1, 0, 0]
    # 3-bit code 5 (0b101) at j = 10: bits 30, 31 take 0b01, bit 32 takes 1
    c = np.zeros((1, 11), np.uint8)
    c[0, 10] = 5
    assert list(deploy.pack_codes(c, 3)[0]) == [0x40000000, 0x1, 0, 0]
    # 4-bit nibbles in order
    assert deploy.pack_codes(np.array([[0xA, 0xB, 0x0, 0xF]], np.uint8), 4)[0, 0] == 0xF0BA


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d_in", [1, 31, 33, 130])
def test_pack_roundtrip(bits, d_in):
    rng = np.random.default_rng(bits * 1000 + d_in)
    codes = rng.integers(0, 1 << bits, (5, d_in)).astype(np.uint8)
    p = deploy.pack_codes(codes, bits)
    assert p.shape == (5, deploy.packed_row_words(d_in, bits))
    np.testing.assert_array_equal(deploy.unpack_codes(p, bits, d_in), codes)


def _processed(d_out=64, d_in=96, blk_in=32, blk_out=0, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((400, d_in)) * np.exp(rng.standard_normal(d_in))
    g = rng.standard_normal((400, d_out)) * np.exp(rng.standard_normal(d_out))
    HX, _, HG = oracle.covariances(None, x.astype(np.float32), g.astype(np.float32))
    W = 0.02 * rng.standard_normal((d_out, d_in))
    si = rng.choice([-1, 1], d_in).astype(np.int8)
    so = rng.choice([-1, 1], d_out).astype(np.int8)
    W2, _, _, _, s_x, s_g = oracle.biip(W, HX, None, HG, si, so, blk_in, blk_out)
    return W, W2, s_x, s_g, si, so, rng


def test_detransform_undoes_biip():
    W, W2, s_x, s_g, si, so, _ = _processed()
    np.testing.assert_allclose(deploy.detransform(W2, s_x, s_g, si, so, 32, 0), W, rtol=0, atol=1e-14)


@pytest.mark.parametrize("bits,group", [(2, 0), (3, 32), (4, 0)])
def test_infer_equals_dense_detransformed_product(bits, group):
    W, W2, s_x, s_g, si, so, rng = _processed(seed=bits)
    n_groups = W2.shape[1] // group if group else 1
    codes = rng.integers(0, 1 << bits, W2.shape).astype(np.uint8)
    scale = rng.uniform(0.01, 0.02, (W2.shape[0], n_groups)).astype(np.float32)
    zero = rng.integers(0, 1 << bits, (W2.shape[0], n_groups)).astype(np.float32)
    Wq = deploy.dequantize(codes, scale, zero, group)
    dense = deploy.detransform(Wq, s_x, s_g, si, so, 32, 0)
    x = rng.standard_normal((3, W2.shape[1]))
    y = deploy.infer(x, deploy.pack_codes(codes, bits), bits, scale, zero, group, s_x, s_g, si, so, 32, 0)
    np.testing.assert_allclose(y, x @ dense.T, rtol=1e-12, atol=1e-12)


def test_dequantize_groups_entrywise():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 8, (3, 12)).astype(np.uint8)
    scale = rng.uniform(0.5, 1.5, (3, 3))
    zero = rng.integers(0, 8, (3, 3)).astype(np.float64)
    Wq = deploy.dequantize(codes, scale, zero, 4)
    for i in range(3):
        for j in range(12):
            assert Wq[i, j] == scale[i, j // 4] * (codes[i, j] - zero[i, j // 4])


def test_infer_of_the_sweep_is_the_detransformed_layer():
    """With the oracle's own sweep on the toy layer, stepwise inference equals
    the product with the de-transformed dequantized matrix."""
    from synth import layer_specs, make_layer
    spec = layer_specs(0)[0]
    L = make_layer(spec, n_tok=256)
    HX, D, HG = oracle.covariances(L["x"], L["xq"], L["g"])
    W2, HX2, D2, HG2, s_x, s_g = oracle.biip(L["W"], HX, D, HG, L["sign_in"], L["sign_out"])
    U = oracle.inv_factor(HX2, 0.01)
    res = oracle.sweep(W2, U, oracle.form_p(D2, U), 4, 0, 128)
    p = deploy.pack_codes(res["codes"], 4)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 256))
    y = deploy.infer(x, p, 4, res["scale"], res["zero"], 0, s_x, s_g, L["sign_in"], L["sign_out"])
    dense = deploy.detransform(res["what"], s_x, s_g, L["sign_in"], L["sign_out"])
    np.testing.assert_allclose(y, x @ dense.T, rtol=1e-9, atol=1e-12)
