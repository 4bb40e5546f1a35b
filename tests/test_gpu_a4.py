"""GPU parity of the product with 2-bit weights and 4-bit activations
(kq_apply_quantized_a4) against oracle/deploy.py (infer_a4).

The activation codes are integers decided in fp32 on both sides, from a
rotated input that the GPU computes in fp32 and the oracle in fp64 then
rounds to fp32, so they are compared by forced replay: at most 1e-4 of them
may differ, each by one level and with the oracle's x2 / s within 1e-4 of
the midpoint between the two levels; the oracle then takes the GPU's codes.
The scales s agree to 1e-6 relative. The output is held to 1e-5 relative
(Frobenius over the batch): the integer product is exact and only the
transforms and the final scalings round.

With the rotation and the output transform reduced to the identity (blocks
of 1, unit signs and scalings) and inputs that are integers of largest
magnitude 7, s = 1 and the GPU's output is the integer product
sum_k q_k a_k - zero sum_k a_k itself: that is checked bit-exactly.
"""
import numpy as np
import pytest

from oracle import deploy
from tests.gpu_util import dev, have_gpu, host, rel_fro

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

if have_gpu():
    import torch

    import post_weight_quantization_amd as kq


def _case(d_out, d_in, rng):
    codes = rng.integers(0, 4, (d_out, d_in)).astype(np.uint8)
    scale = rng.uniform(0.005, 0.02, d_out).astype(np.float32)
    zero = rng.integers(0, 4, d_out).astype(np.float32)
    s_x = np.exp(rng.normal(0, 0.5, d_in)).astype(np.float32)
    s_g = np.exp(rng.normal(0, 0.5, d_out)).astype(np.float32)
    si = rng.choice([-1, 1], d_in).astype(np.int8)
    so = rng.choice([-1, 1], d_out).astype(np.int8)
    return codes, scale, zero, s_x, s_g, si, so


def _gpu(codes, scale, zero, s_x, s_g, si, so, x, clip=1.0, bi=0, bo=0):
    batch, d_in = x.shape
    packed = kq.kq_pack_codes(dev(codes), 2)
    ac = torch.empty(batch, d_in, dtype=torch.int8, device="cuda")
    asc = torch.empty(batch, dtype=torch.float32, device="cuda")
    y = kq.kq_apply_quantized_a4(packed, dev(scale), dev(zero), dev(s_x), dev(s_g), dev(si), dev(so),
                                 dev(x), clip, bi, bo, act_codes=ac, act_scale=asc)
    return host(y), host(ac), host(asc)


def _check(codes, scale, zero, s_x, s_g, si, so, x, clip=1.0, bi=0, bo=0):
    y, ac, asc = _gpu(codes, scale, zero, s_x, s_g, si, so, x, clip, bi, bo)
    packed = deploy.pack_codes(codes, 2)
    own = deploy.infer_a4(x, packed, 2, scale, zero, 0, s_x, s_g, si, so, bi, bo, clip=clip)
    diff = ac != own["q"]
    n = int(diff.sum())
    assert n <= max(1, int(1e-4 * ac.size)), f"{n} activation codes differ"
    if n:
        assert np.all(np.abs(ac[diff].astype(int) - own["q"][diff].astype(int)) == 1)
        mid = 0.5 * (ac[diff].astype(np.float64) + own["q"][diff])
        assert np.max(np.abs(own["t"][diff] - mid)) <= 1e-4
    np.testing.assert_allclose(asc, own["s"], rtol=1e-6, atol=0)
    want = deploy.infer_a4(x, packed, 2, scale, zero, 0, s_x, s_g, si, so, bi, bo, clip=clip,
                           forced_act=ac)
    err = rel_fro(y, want["y"])
    assert err < 1e-5, err
    return y, ac, asc, err


# one super-step; a ragged K range (3 super-steps); a vector split over
# transform chunks (unfused quantization); a whole 8192 vector in one chunk;
# batches of 1, 16 (one full tile), 17 and 40 (a partial tile); many tiles,
# where a workgroup takes 128 rows (the last row block ragged at 2100);
# grids of >= 256 workgroups of 256 rows x 32 vectors take the GEMM (ragged
# rows and vectors at 2100 x 930, whole blocks at 2048 x 1024); a long K
# with several vector tiles on the K-split product (2100 x 24576, batch 120)
@pytest.mark.parametrize("d_out,d_in,batch,bi,bo,clip", [
    (256, 512, 1, 0, 0, 1.0), (260, 1536, 17, 512, 0, 0.9), (128, 4096, 16, 0, 0, 1.0),
    (64, 12288, 5, 4096, 32, 0.8), (96, 8192, 40, 0, 0, 1.0), (512, 2048, 3, 256, 128, 1.0),
    (4096, 1024, 256, 256, 0, 0.9), (2100, 1024, 600, 0, 0, 1.0), (2100, 512, 930, 0, 0, 1.0),
    (2048, 1536, 1024, 512, 0, 0.9), (2100, 24576, 120, 0, 0, 1.0)])
def test_a4_against_oracle(d_out, d_in, batch, bi, bo, clip):
    rng = np.random.default_rng(d_out + d_in + batch)
    c = _case(d_out, d_in, rng)
    x = (rng.standard_normal((batch, d_in)) * np.exp(rng.normal(0, 1, (batch, 1)))).astype(np.float32)
    _check(*c, x, clip, bi, bo)


@pytest.mark.parametrize("d_out,d_in,batch", [(260, 1536, 1), (64, 512, 16), (200, 2560, 17),
                                              (8, 4096, 40), (2100, 1024, 930), (2100, 24576, 120)])
def test_a4_integer_product_bit_exact(d_out, d_in, batch):
    """Identity transforms and integer inputs of largest magnitude 7: y is
    sum_k q_k a_k - zero sum_k a_k exactly."""
    rng = np.random.default_rng(3 * d_in + batch)
    codes = rng.integers(0, 4, (d_out, d_in)).astype(np.uint8)
    zero = rng.integers(0, 4, d_out).astype(np.float32)
    a = rng.integers(-8, 8, (batch, d_in)).astype(np.float32)
    a[:, 7] = 7.0
    a = np.clip(a, -7, 7)  # largest magnitude exactly 7: s = 1
    ones_i, ones_o = np.ones(d_in, np.float32), np.ones(d_out, np.float32)
    y, ac, asc = _gpu(codes, np.ones(d_out, np.float32), zero, ones_i, ones_o, np.ones(d_in, np.int8),
                      np.ones(d_out, np.int8), a, 1.0, 1, 1)
    np.testing.assert_array_equal(asc, np.ones(batch, np.float32))
    np.testing.assert_array_equal(ac, a.astype(np.int8))
    exact = a.astype(np.float64) @ codes.T.astype(np.float64) - a.sum(1)[:, None] * zero[None, :]
    np.testing.assert_array_equal(y, exact.astype(np.float32))


def test_a4_degenerate_vectors_and_repeat_calls():
    """An all-zero vector (s = 0, codes 0, y = 0), vectors at 1e-30 and 1e30,
    and a second call after a larger one giving the same result."""
    rng = np.random.default_rng(11)
    c = _case(128, 1024, rng)
    x = rng.standard_normal((4, 1024)).astype(np.float32)
    x[0] = 0.0
    x[1] *= 1e-30
    x[2] *= 1e30
    big = _case(300, 2048, rng)
    _gpu(*big, rng.standard_normal((33, 2048)).astype(np.float32))
    y, ac, asc, _ = _check(*c, x)
    assert asc[0] == 0 and not ac[0].any() and not y[0].any()
    y2, ac2, asc2 = _gpu(*c, x)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(ac2, ac)


def test_a4_close_to_the_weight_only_product():
    """Quantizing the activation moves the output by no more than the
    activation error allows: |W^' (x2 - s a)| <= |W^'| s / 2 per vector, with
    the orthogonal transforms and the diagonal scalings around it."""
    rng = np.random.default_rng(5)
    c = _case(256, 2048, rng)
    codes, scale, zero, s_x, s_g, si, so = c
    x = rng.standard_normal((3, 2048)).astype(np.float32)
    y, ac, asc = _gpu(*c, x)
    packed = kq.kq_pack_codes(dev(codes), 2)
    yw = host(kq.kq_apply_quantized(packed, 2, dev(scale[:, None]), dev(zero[:, None]), 0, dev(s_x),
                                    dev(s_g), dev(si), dev(so), dev(x)))
    Wq = deploy.dequantize(codes, scale, zero)
    bound = np.linalg.norm(Wq, 2) * 0.5 * asc * np.sqrt(2048) / np.min(s_g)
    assert np.all(np.linalg.norm(y - yw, axis=1) <= bound)
    assert rel_fro(y, yw) < 0.3


@pytest.mark.slow
@pytest.mark.parametrize("d_out,d_in,batch", [(4096, 4096, 16), (8192, 28672, 16), (11008, 4096, 33),
                                              (8192, 28672, 256), (8192, 28672, 64)])
def test_a4_full_size(d_out, d_in, batch):
    rng = np.random.default_rng(d_out + batch)
    c = _case(d_out, d_in, rng)
    x = rng.standard_normal((batch, d_in)).astype(np.float32)
    print(f"[a4 full] {d_out}x{d_in} batch {batch}", flush=True)
    *_, err = _check(*c, x, 0.9)
    print(f"[a4 full] rel {err:.3g}", flush=True)
