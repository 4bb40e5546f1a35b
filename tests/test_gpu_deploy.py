"""GPU parity of inference with the quantized layer (packing and the product
y = S_G^-1 U^T W^' V S_X^-1 x) against oracle/deploy.py.

Packing is integer work: bit-exact. The product applies the transforms to
the vectors in fp32; 2-, 4- and 8-bit codes multiply a 23-bit fixed-point
form of each 32-value chunk of the transformed input in integer dot
products (each value off by at most 2^-23 of the chunk's largest, about
fp32's own rounding of that value), 3-bit codes multiply in fp32. Against
the fp64 reference it is held to 1e-5 relative (Frobenius over the batch),
the size of fp32 rounding over sums of d_in terms.
"""
import numpy as np
import pytest

from oracle import deploy
from tests.gpu_util import dev, have_gpu, host, rel_fro, tile_rel_fro

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

if have_gpu():
    import torch

    import post_weight_quantization_amd as kq
    import post_weight_quantization_amd._native as N


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d_out,d_in", [(7, 33), (64, 4096), (3, 11008)])
def test_pack_bit_exact(bits, d_out, d_in):
    rng = np.random.default_rng(bits + d_in)
    codes = rng.integers(0, 1 << bits, (d_out, d_in)).astype(np.uint8)
    got = host(kq.kq_pack_codes(dev(codes), bits)).view(np.uint32)
    np.testing.assert_array_equal(got, deploy.pack_codes(codes, bits))


def _case(d_out, d_in, bits, group, rng):
    ng = d_in // group if group else 1
    codes = rng.integers(0, 1 << bits, (d_out, d_in)).astype(np.uint8)
    scale = rng.uniform(0.005, 0.02, (d_out, ng)).astype(np.float32)
    zero = rng.integers(0, 1 << bits, (d_out, ng)).astype(np.float32)
    s_x = np.exp(rng.normal(0, 0.5, d_in)).astype(np.float32)
    s_g = np.exp(rng.normal(0, 0.5, d_out)).astype(np.float32)
    si = rng.choice([-1, 1], d_in).astype(np.int8)
    so = rng.choice([-1, 1], d_out).astype(np.int8)
    return codes, scale, zero, s_x, s_g, si, so


def _run(codes, scale, zero, s_x, s_g, si, so, bits, group, x, bi=0, bo=0):
    packed = kq.kq_pack_codes(dev(codes), bits)
    y = kq.kq_apply_quantized(packed, bits, dev(scale), dev(zero), group, dev(s_x), dev(s_g), dev(si),
                              dev(so), dev(x), bi, bo)
    want = deploy.infer(x, deploy.pack_codes(codes, bits), bits, scale, zero, group, s_x, s_g, si, so,
                        bi, bo)
    return host(y), want


@pytest.mark.parametrize("bits,group,bi,bo,batch", [
    (2, 0, 0, 0, 1), (3, 128, 0, 0, 3), (4, 0, 128, 64, 5), (8, 128, 0, 32, 8), (2, 128, 256, 0, 4)])
def test_apply_against_oracle(bits, group, bi, bo, batch):
    rng = np.random.default_rng(bits * 7 + batch)
    c = _case(256, 512, bits, group, rng)
    x = rng.standard_normal((batch, 512)).astype(np.float32)
    got, want = _run(*c, bits, group, x, bi, bo)
    assert rel_fro(got, want) < 1e-5
    # and 32 outputs at a time, vector by vector: one wrong segment of small
    # outputs cannot hide behind the rest
    for v in range(batch):
        assert tile_rel_fro(got[v:v + 1], want[v:v + 1], 32) < 1e-4, v


def test_apply_on_the_pipeline_output():
    """Codes, grids and scalings straight from the GPU pipeline on the toy layer."""
    from synth import layer_specs, make_layer
    spec = layer_specs(0)[0]
    L = make_layer(spec)
    HX, D, HG = kq.kq_accumulate_cov(dev(L["x"]), dev(L["xq"]), dev(L["g"]), 1.0 / spec.n_tok, 0.0)
    W = dev(L["W"])
    s_x, s_g = kq.kq_biip(W, HX, D, HG, dev(L["sign_in"]), dev(L["sign_out"]))
    U = kq.kq_cholesky_inv(HX, spec.damp)
    codes, scale, zero = kq.kq_gptaq_quantize(W, U, D, spec.bits, spec.group)
    x = np.random.default_rng(1).standard_normal((2, spec.d_in)).astype(np.float32)
    y = kq.kq_apply_quantized(kq.kq_pack_codes(codes, spec.bits), spec.bits, scale, zero, 0, s_x, s_g,
                              dev(L["sign_in"]), dev(L["sign_out"]), dev(x))
    want = deploy.infer(x, deploy.pack_codes(host(codes), spec.bits), spec.bits, host(scale),
                        host(zero), 0, host(s_x), host(s_g), L["sign_in"], L["sign_out"])
    assert rel_fro(host(y), want) < 1e-5
    # and the product with the de-transformed dequantized layer the sweep returned
    dense = deploy.detransform(host(W), host(s_x), host(s_g), L["sign_in"], L["sign_out"])
    assert rel_fro(host(y), x @ dense.T) < 1e-5


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("group,batch", [(0, 1), (128, 2), (0, 3), (128, 6)])
def test_apply_ragged(bits, group, batch):
    # 260 rows: the last row group of a wave is partial; 2176 columns = 68
    # chunks of 32: two K tiles of 64 lanes, the second with 4 active lanes;
    # batches 1, 2, 3 and 6 take every vector-count variant (6 = 4 + 2)
    rng = np.random.default_rng(1000 * bits + 10 * batch + group)
    c = _case(260, 2176, bits, group, rng)
    x = rng.standard_normal((batch, 2176)).astype(np.float32)
    got, want = _run(*c, bits, group, x)
    assert rel_fro(got, want) < 1e-5
    for v in range(batch):
        assert tile_rel_fro(got[v:v + 1], want[v:v + 1], 32) < 1e-4, v


@pytest.mark.parametrize("batch", [3, 4, 5, 6, 7, 9])
def test_apply_matrix_core_launch_splits(batch):
    # 2-bit per-row codes with d_in a multiple of 512 take the matrix-core
    # product: one launch per four vectors, then one for the 1-3 left over
    # (batch 9 = 4 + 4 + 1). 260 rows end in a partial 16-row tile; 1536
    # columns are 3 super-steps, so the two-per-range launches end in a
    # ragged range
    rng = np.random.default_rng(500 + batch)
    c = _case(260, 1536, 2, 0, rng)
    x = rng.standard_normal((batch, 1536)).astype(np.float32)
    x[batch // 2] *= 1e-3  # vectors of different magnitudes share a launch
    got, want = _run(*c, 2, 0, x, bi=512, bo=0)
    for v in range(batch):
        assert rel_fro(got[v:v + 1], want[v:v + 1]) < 1e-5, v


@pytest.mark.parametrize("d_out,d_in,batch", [(4100, 8704, 5), (4100, 8704, 1), (1028, 17408, 3)])
def test_apply_matrix_core_k_groups(d_out, d_in, batch):
    # 17 and 34 super-steps split into 17 groups of columns, each group's
    # partial product in its own plane; 4100 rows take 128-row workgroups
    # (a wave streams 8 row tiles through its ring, the last workgroup 4
    # rows), 1028 rows 64-row workgroups (the last 4 rows)
    rng = np.random.default_rng(d_in + batch)
    c = _case(d_out, d_in, 2, 0, rng)
    x = rng.standard_normal((batch, d_in)).astype(np.float32)
    got, want = _run(*c, 2, 0, x)
    for v in range(batch):
        assert rel_fro(got[v:v + 1], want[v:v + 1]) < 1e-5, v


def test_apply_matrix_core_workspace_reuse():
    # one workspace, sized for 6 vectors, serves a 6-vector call and then a
    # 2-vector call: the K groups' partial planes are laid out by the
    # call's own batch, and every entry the second call reads is its own
    d_out, d_in = 4100, 8704
    rng = np.random.default_rng(91)
    codes, scale, zero, s_x, s_g, si, so = _case(d_out, d_in, 2, 0, rng)
    packed = kq.kq_pack_codes(dev(codes), 2)
    ws = torch.empty(kq.kq_workspace_size(N.KQ_OP_APPLY_QUANTIZED, d_out, d_in, 6), dtype=torch.uint8,
                     device="cuda")
    for batch in (6, 2):
        x = rng.standard_normal((batch, d_in)).astype(np.float32)
        y = kq.kq_apply_quantized(packed, 2, dev(scale), dev(zero), 0, dev(s_x), dev(s_g), dev(si),
                                  dev(so), dev(x), ws=ws)
        want = deploy.infer(x, deploy.pack_codes(codes, 2), 2, scale, zero, 0, s_x, s_g, si, so)
        for v in range(batch):
            assert rel_fro(host(y)[v:v + 1], want[v:v + 1]) < 1e-5, (batch, v)


@pytest.mark.parametrize("bits", [2, 3, 8])
def test_apply_dynamic_range(bits):
    # Hadamard blocks of 32 keep every 32-column chunk of the transformed
    # input at its own magnitude: chunks from 1e-6 to 1e6, and all-zero
    # chunks, so each chunk's own exponent in the integer products matters
    rng = np.random.default_rng(77 + bits)
    d_out, d_in, batch = 128, 4096, 3
    c = _case(d_out, d_in, bits, 0, rng)
    mag = 10.0 ** rng.uniform(-6, 6, (batch, d_in // 32))
    mag[:, ::7] = 0.0
    x = (rng.standard_normal((batch, d_in)) * np.repeat(mag, 32, axis=1)).astype(np.float32)
    got, want = _run(*c, bits, 0, x, bi=32, bo=0)
    assert rel_fro(got, want) < 1e-5
    # rows are dominated by the largest chunks: check a small-input vector too
    x2 = (rng.standard_normal((1, d_in)) * 1e-30).astype(np.float32)
    got2, want2 = _run(*c, bits, 0, x2, bi=32, bo=0)
    assert rel_fro(got2, want2) < 1e-5


@pytest.mark.parametrize("bits,group", [(2, 0), (3, 128), (4, 0)])
def test_apply_one_chunk_per_vector(bits, group):
    """Each vector holds a single nonzero 32-column chunk of the rotated input
    (Hadamard blocks of 32), at magnitudes from 1e-6 to 1e6 or zero, so every
    output of that vector comes from that chunk alone and is checked on its
    own scale: per vector, and per 32-entry run of outputs."""
    rng = np.random.default_rng(91 + bits)
    d_out, d_in = 128, 1024
    c = _case(d_out, d_in, bits, group, rng)
    mags = [0.0, 1e-6, 1e-3, 1.0, 1e3, 1e6]
    chunks = rng.choice(d_in // 32, len(mags), replace=False)
    x = np.zeros((len(mags), d_in), np.float32)
    for v, (m, k) in enumerate(zip(mags, chunks)):
        x[v, 32 * k:32 * k + 32] = m * rng.standard_normal(32)
    got, want = _run(*c, bits, group, x, bi=32, bo=0)
    assert np.all(got[0] == 0.0)
    for v in range(1, len(mags)):
        assert rel_fro(got[v], want[v]) < 1e-5, (v, mags[v])
        assert tile_rel_fro(got[v], want[v], 32) < 1e-4, (v, mags[v])


@pytest.mark.slow
@pytest.mark.parametrize("d_out,d_in,bits,group", [(4096, 4096, 2, 0), (11008, 4096, 3, 128),
                                                   (8192, 28672, 2, 0)])
def test_apply_full_size(d_out, d_in, bits, group):
    rng = np.random.default_rng(d_in)
    c = _case(d_out, d_in, bits, group, rng)
    x = rng.standard_normal((4, d_in)).astype(np.float32)
    got, want = _run(*c, bits, group, x)
    err = rel_fro(got, want)
    tile = max(tile_rel_fro(got[v], want[v], 256) for v in range(got.shape[0]))
    print(f"{d_out}x{d_in} {bits}-bit: rel {err:.3g}, worst 256-output run {tile:.3g}")
    assert err < 1e-5 and tile < 1e-4
