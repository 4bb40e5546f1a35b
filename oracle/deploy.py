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
