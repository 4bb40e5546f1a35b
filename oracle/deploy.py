"""fp64 reference of inference with a KronQ-quantized layer (test infrastructure only).

[GS] KronQ explainer on gist.science, "Limitazioni": at inference the only
overhead left is the orthogonal transforms, the same as QuIP#'s. The
processed layer W' = U S_G W S_X V^T ([KS] Method, BiIP scaling and
rotation equations) is stored quantized; the original basis is recovered as
    W^ = S_G^-1 U^T W^' V S_X^-1,
so a product with an input x never forms W^:
    y = W^ x = S_G^-1 U^T (W^' (V (S_X^-1 x))).
Here U = blockdiag(H_b / sqrt b) diag(sign_out) and V likewise on the input
side (the reading of the random Hadamard used by biip()), so
U^T = diag(sign_out) blockdiag(H_b / sqrt b).

Packing (a storage format of this library, not of the method): each row of
codes is a little-endian bit stream, code j in bits [b j, b j + b) of the
row, in 32-bit words; rows are padded to a multiple of 4 words (16 bytes).
"""
from __future__ import annotations

import numpy as np

from .kronq import apply_hadamard_left, hadamard_block


def packed_row_words(d_in: int, bits: int) -> int:
    """32-bit words per packed row: ceil(d_in * bits / 32), rounded up to 4."""
    w = (d_in * bits + 31) // 32
    return (w + 3) // 4 * 4


def pack_codes(codes, bits: int) -> np.ndarray:
    """Codes (d_out x d_in, values < 2^bits) -> packed words (d_out x row_words)."""
    codes = np.asarray(codes)
    d_out, d_in = codes.shape
    if np.any(codes >= (1 << bits)):
        raise ValueError("code out of range")
    nw = packed_row_words(d_in, bits)
    out = np.zeros((d_out, nw), dtype=np.uint64)
    for j in range(d_in):
        bit = bits * j
        w, sh = bit // 32, bit % 32
        v = codes[:, j].astype(np.uint64) << np.uint64(sh)
        out[:, w] |= v & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:
            out[:, w + 1] |= v >> np.uint64(32)
    return out.astype(np.uint32)


def unpack_codes(packed, bits: int, d_in: int) -> np.ndarray:
    """Inverse of pack_codes."""
    p = np.asarray(packed, dtype=np.uint64)
    d_out = p.shape[0]
    out = np.zeros((d_out, d_in), dtype=np.uint8)
    mask = np.uint64((1 << bits) - 1)
    for j in range(d_in):
        bit = bits * j
        w, sh = bit // 32, bit % 32
        v = p[:, w] >> np.uint64(sh)
        if sh + bits > 32:
            v |= p[:, w + 1] << np.uint64(32 - sh)
        out[:, j] = (v & mask).astype(np.uint8)
    return out


def dequantize(codes, scale, zero, group: int = 0) -> np.ndarray:
    """W^'[i][j] = scale[i][g] (q[i][j] - zero[i][g]), g = j // group (one grid per row if 0)."""
    q = np.asarray(codes, np.float64)
    sc = np.asarray(scale, np.float64)
    zr = np.asarray(zero, np.float64)
    if sc.ndim == 1:
        sc, zr = sc[:, None], zr[:, None]
    gs = group or q.shape[1]
    return np.repeat(sc, gs, axis=1)[:, :q.shape[1]] * (q - np.repeat(zr, gs, axis=1)[:, :q.shape[1]])


def detransform(Wp, s_x, s_g, sign_in, sign_out, blk_in: int = 0, blk_out: int = 0) -> np.ndarray:
    """W = S_G^-1 U^T W' V S_X^-1: the inverse of biip()'s transform of W."""
    Wp = np.asarray(Wp, np.float64)
    d_out, d_in = Wp.shape
    bi = blk_in or hadamard_block(d_in)
    bo = blk_out or hadamard_block(d_out)
    so = np.asarray(sign_out, np.float64)
    si = np.asarray(sign_in, np.float64)
    # U^T M = diag(sign_out) blockdiag(H/sqrt b) M
    A = so[:, None] * apply_hadamard_left(Wp, np.ones(d_out), bo)
    # (M V) = (V^T M^T)^T, V^T = diag(sign_in) blockdiag(H/sqrt b)
    B = (si[:, None] * apply_hadamard_left(A.T, np.ones(d_in), bi)).T
    return B / np.asarray(s_g, np.float64)[:, None] / np.asarray(s_x, np.float64)[None, :]


def infer(x, packed, bits: int, scale, zero, group: int, s_x, s_g, sign_in, sign_out,
          blk_in: int = 0, blk_out: int = 0) -> np.ndarray:
    """y = S_G^-1 U^T (W^' (V (S_X^-1 x))) for a batch x (B x d_in), step by step."""
    x = np.atleast_2d(np.asarray(x, np.float64))
    d_in = x.shape[1]
    d_out = np.asarray(packed).shape[0]
    bi = blk_in or hadamard_block(d_in)
    bo = blk_out or hadamard_block(d_out)
    x1 = x / np.asarray(s_x, np.float64)[None, :]
    x2 = apply_hadamard_left(x1.T, sign_in, bi)                      # d_in x B
    Wq = dequantize(unpack_codes(packed, bits, d_in), scale, zero, group)
    y1 = Wq @ x2                                                     # d_out x B
    y2 = np.asarray(sign_out, np.float64)[:, None] * apply_hadamard_left(y1, np.ones(d_out), bo)
    return (y2 / np.asarray(s_g, np.float64)[:, None]).T


# ---------------------------------------------------------------------------
# Weights and activations both quantized (the W2A4 setting).
#
# [GS] KronQ explainer, "Quantizzazione di Pesi e Attivazioni": for the
# weight-and-activation results the activations follow the QuaRot recipe.
# The pages give no more than that. Readings taken here:
#   * the activation is quantized where the rotation leaves it, i.e. the
#     rotated input x2 = V S_X^-1 x that the quantized rows W^' act on
#     (the rotation spreads outliers before rounding);
#   * one grid per vector (per token), symmetric, round to nearest (ties to
#     even), s = clip * max_k |x2_k| / (2^(b-1) - 1), q = clamp(rint(x2 / s),
#     -2^(b-1), 2^(b-1) - 1); the clipping ratio is the caller's; an all-zero
#     vector has s = 0 and q = 0;
#   * the integer decision is taken in fp32 (x2 rounded to fp32, then the
#     max, the product with clip, the division by 2^(b-1) - 1 and the division
#     x2 / s each rounded to fp32), the precision of the kernels.


def quantize_activations(x2, bits: int = 4, clip: float = 1.0, forced=None):
    """Per-vector symmetric RTN of x2 (B x d_in). Returns dict(q int8, s fp32
    per vector, t = x2 / s in fp32: the values that were rounded).

    forced: codes to use instead of the rounding (each must be within 1e-4 of
    a rounding boundary of t where it differs; the caller checks that)."""
    x = np.atleast_2d(np.asarray(x2, np.float64)).astype(np.float32)
    qmax = (1 << (bits - 1)) - 1
    mx = np.max(np.abs(x), axis=1)
    s = (np.float32(clip) * mx).astype(np.float32) / np.float32(qmax)
    s = s.astype(np.float32)
    t = np.zeros_like(x)
    nz = s > 0
    t[nz] = x[nz] / s[nz, None]
    q = np.clip(np.rint(t), -qmax - 1, qmax).astype(np.int8)
    if forced is not None:
        q = np.asarray(forced, np.int8).reshape(q.shape)
    return {"q": q, "s": s, "t": t}


def rotate_input(x, s_x, sign_in, blk_in: int = 0) -> np.ndarray:
    """x2 = V S_X^-1 x for a batch (B x d_in), in fp64."""
    x = np.atleast_2d(np.asarray(x, np.float64))
    bi = blk_in or hadamard_block(x.shape[1])
    x1 = x / np.asarray(s_x, np.float64)[None, :]
    return apply_hadamard_left(x1.T, sign_in, bi).T


def infer_a4(x, packed, bits: int, scale, zero, group: int, s_x, s_g, sign_in, sign_out,
             blk_in: int = 0, blk_out: int = 0, act_bits: int = 4, clip: float = 1.0,
             forced_act=None) -> dict:
    """y = S_G^-1 U^T (W^' (s q)) with (q, s) the per-vector quantization of
    x2 = V S_X^-1 x, step by step (fp64 apart from the fp32 decision).
    Returns dict(y, q, s, t)."""
    x2 = rotate_input(x, s_x, sign_in, blk_in)
    qa = quantize_activations(x2, act_bits, clip, forced_act)
    d_in = x2.shape[1]
    d_out = np.asarray(packed).shape[0]
    bo = blk_out or hadamard_block(d_out)
    xa = qa["s"].astype(np.float64)[:, None] * qa["q"].astype(np.float64)   # B x d_in
    Wq = dequantize(unpack_codes(packed, bits, d_in), scale, zero, group)
    y1 = Wq @ xa.T                                                            # d_out x B
    y2 = np.asarray(sign_out, np.float64)[:, None] * apply_hadamard_left(y1, np.ones(d_out), bo)
    return {"y": (y2 / np.asarray(s_g, np.float64)[:, None]).T, **qa}
