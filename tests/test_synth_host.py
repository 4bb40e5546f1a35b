"""The seeded input recipe (CPU): the generator that both the oracle and the
HIP path read draws what the workload description states, reproducibly and
chunk by chunk.

The recipe stands in for the pages' LLaMA calibration sets (KronQ summary,
hyper.ai, Experiments): per-channel activation scales LogNormal(0, 1) with the
first channels scaled x20, X~ = X + N(0, (0.01 sigma)^2), output-gradient
scales LogNormal(0, 2) (a diag(H_G) spread over orders of magnitude, as the
Method section's figure shows), W ~ N(0, 0.02^2), +-1 signs, bf16 by
round-to-nearest-even. The statistical bounds below are several standard
errors wide for the sample sizes used.
"""
from dataclasses import replace

import numpy as np
import pytest

from synth import CHUNK, bf16_bits_to_f32, layer_specs, make_layer, token_chunk


def _bf16_nearest_even(x):
    """Nearest bf16 by the significand (8 significant bits, rint = ties to
    even), as fp32 values: another route than the generator's bit arithmetic."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8).astype(np.float32)


def test_reproducible_and_chunked():
    spec = replace(layer_specs(1)[0], d_out=384, d_in=512)   # narrower, same streams
    a = make_layer(spec, n_tok=CHUNK + 300, threads=1)
    b = make_layer(spec, n_tok=CHUNK + 300, threads=4)
    for k in ("x", "xq", "g", "W", "sign_in", "sign_out"):
        np.testing.assert_array_equal(a[k], b[k])
    # a prefix is the same tokens; chunk c is rows [c CHUNK, (c + 1) CHUNK)
    short = make_layer(spec, n_tok=100, threads=1)
    np.testing.assert_array_equal(short["x"], a["x"][:100])
    np.testing.assert_array_equal(token_chunk(spec, "xq", 1, 300), a["xq"][CHUNK:])
    np.testing.assert_array_equal(token_chunk(spec, "g", 0, 50), a["g"][:50])
    # the streams differ from each other
    assert not np.array_equal(a["x"][:, :16], a["xq"][:, :16])
    assert a["x"].dtype == np.uint16 and a["x"].shape == (CHUNK + 300, 512)
    assert a["g"].shape == (CHUNK + 300, 384) and a["W"].shape == (384, 512)
    assert a["W"].dtype == np.float32


def test_bf16_is_the_nearest_even_rounding_of_the_fp32_draw():
    spec = layer_specs(1)[0]
    f32 = replace(spec, dtype="f32")
    for which in ("x", "xq", "g"):
        raw = token_chunk(f32, which, 0, 256)
        bits = token_chunk(spec, which, 0, 256)
        np.testing.assert_array_equal(bf16_bits_to_f32(bits), _bf16_nearest_even(raw))


def test_activation_recipe():
    spec = layer_specs(1)[0]
    f32 = replace(spec, dtype="f32")
    n = CHUNK
    x = token_chunk(f32, "x", 0, n).astype(np.float64)
    xq = token_chunk(f32, "xq", 0, n).astype(np.float64)
    rms = np.sqrt(np.mean(x * x, axis=0))
    # per-channel scales: LogNormal(0, 1), the first 16 channels x20
    ls = np.log(rms)
    assert abs(np.mean(ls[16:])) < 0.1 and abs(np.std(ls[16:]) - 1.0) < 0.06
    assert abs(np.mean(ls[:16]) - np.log(20.0)) < 1.0
    assert np.min(rms[:16]) > 20 * np.exp(-3.5)
    # X~ - X is N(0, (0.01 sigma)^2) channel by channel, independent of X
    dn = (xq - x) / rms[None, :]
    assert np.sqrt(np.mean(dn * dn)) == pytest.approx(0.01, rel=0.02)
    corr = np.mean(dn * (x / rms[None, :])) / 0.01
    assert abs(corr) < 0.01
    # toy layer: fp32, 4 outlier channels
    toy = layer_specs(0)[0]
    t = make_layer(toy, threads=1)
    assert t["x"].dtype == np.float32 and t["x"].shape == (1024, 256)
    tr = np.sqrt(np.mean(t["x"].astype(np.float64) ** 2, axis=0))
    assert np.median(tr[:4]) > 5 * np.median(tr[4:])


def test_gradient_weight_and_sign_recipe():
    spec = layer_specs(1)[0]
    f32 = replace(spec, dtype="f32")
    g = token_chunk(f32, "g", 0, CHUNK).astype(np.float64)
    lt = np.log(np.sqrt(np.mean(g * g, axis=0)))
    assert abs(np.mean(lt)) < 0.15 and abs(np.std(lt) - 2.0) < 0.1   # LogNormal(0, 2)
    L = make_layer(spec, n_tok=8, threads=1)
    W = L["W"].astype(np.float64)
    assert np.std(W) == pytest.approx(0.02, rel=0.01) and abs(np.mean(W)) < 1e-4
    for s in (L["sign_in"], L["sign_out"]):
        assert s.dtype == np.int8 and set(np.unique(s)) == {-1, 1}
        assert abs(np.mean(s)) < 0.05


def test_streams_shared_and_separate_within_a_block():
    """Sublayers reading the same input share X (q, k and v of the decoder
    block); each sublayer has its own G, W and signs."""
    q, k, v, o = layer_specs(4)[:4]
    xq_ = token_chunk(q, "x", 0, 64)
    np.testing.assert_array_equal(xq_, token_chunk(k, "x", 0, 64))
    np.testing.assert_array_equal(xq_, token_chunk(v, "x", 0, 64))
    assert not np.array_equal(xq_, token_chunk(o, "x", 0, 64))
    assert not np.array_equal(token_chunk(k, "g", 0, 64), token_chunk(v, "g", 0, 64))
    lk, lv = make_layer(k, n_tok=1, threads=1), make_layer(v, n_tok=1, threads=1)
    assert not np.array_equal(lk["W"], lv["W"])
    assert not np.array_equal(lk["sign_out"], lv["sign_out"])
