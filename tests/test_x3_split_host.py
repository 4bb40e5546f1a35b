"""Host checks of the arithmetic behind the fp32 products on the bf16 matrix
cores (the three-term split of the GPU GEMM), written independently of the
device code: every fp32 value is the exact sum of three bf16 values taken by
truncation, and the six term products that the kernel keeps give a dot
product within fp32 rounding of the exact one."""
import numpy as np


def bf16_trunc(x):
    """The bf16 value whose bits are the top 16 of x's fp32 bits."""
    return (np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def split3(x):
    x = np.asarray(x, np.float32)
    h = bf16_trunc(x)
    r1 = (x - h).astype(np.float32)
    m = bf16_trunc(r1)
    r2 = (r1 - m).astype(np.float32)
    l = bf16_trunc(r2)
    return h, m, l, r2


def test_split_is_exact():
    """Exact wherever the two residuals stay normal fp32 numbers (|x| above
    about 2^-100; the solver's operands are many orders of magnitude larger)."""
    rng = np.random.default_rng(0)
    tiny = (rng.standard_normal(1000) * 1e-25).astype(np.float32)
    tiny = tiny[np.abs(tiny) > 2.0 ** -100]
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        tiny,
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0, 1 / 3, np.float32(np.pi)], np.float32),
    ])
    h, m, l, r2 = split3(x)
    # the third remainder is itself a bf16 value, so nothing is dropped
    assert np.array_equal(l, r2)
    s = h.astype(np.float64) + m.astype(np.float64) + l.astype(np.float64)
    assert np.array_equal(s, x.astype(np.float64))
    # each term has at most 8 significant bits: its low 16 fp32 bits are 0
    for t in (h, m, l):
        assert not np.any(t.view(np.uint32) & np.uint32(0xFFFF))


def test_six_term_products_within_fp32_rounding():
    rng = np.random.default_rng(1)
    K = 512
    A = rng.standard_normal((32, K)).astype(np.float32)
    B = (rng.standard_normal((K, 32)) * np.exp(rng.standard_normal((K, 1)))).astype(np.float32)
    ah, am, al, _ = split3(A)
    bh, bm, bl, _ = split3(B)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    terms = [(al, bh), (am, bm), (ah, bl), (am, bh), (ah, bm), (ah, bh)]
    acc = np.zeros((32, 32), np.float32)
    for k in range(0, K, 16):  # one 16-deep MFMA step: bf16 x bf16 products exact, fp32 sum
        for a, b in terms:
            part = a[:, k:k + 16].astype(np.float64) @ b[k:k + 16].astype(np.float64)
            acc = (acc + part.astype(np.float32)).astype(np.float32)
    scale = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64)
    err = np.max(np.abs(acc - exact) / scale)
    # the dropped products weigh at most 2^-24 of the leading one; with 6 x
    # K/16 fp32 additions the bound is a few hundred ulps relative to scale
    assert err < 2.0 ** -24 * 6 * (K // 16)
    # and dropping a term the kernel keeps is visibly worse
    acc2 = np.zeros((32, 32), np.float32)
    for k in range(0, K, 16):
        for a, b in terms[1:]:
            part = a[:, k:k + 16].astype(np.float64) @ b[k:k + 16].astype(np.float64)
            acc2 = (acc2 + part.astype(np.float32)).astype(np.float32)
    assert np.max(np.abs(acc2 - exact) / scale) > 10 * err
