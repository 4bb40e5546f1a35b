"""Thin torch binding of the C ABI in include/kq.h.

Each function has the name of the C entry point it calls and only marshals
arguments: it reads shapes and device pointers from torch tensors, allocates
outputs and scratch memory with torch when the caller passes none, and passes
the current HIP stream. Every step of the computation runs in libkq's kernels.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _native as N
from ._native import KQError, check  # noqa: F401


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _expect(t, shape, dtype, name):
    """Shape and dtype of a tensor handed to the library (it sees raw pointers)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape) and t.numel() != int(np.prod(shape)):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")


def kq_workspace_size(op: int, d_out: int, d_in: int, n_tok: int = 0, dtype: int = N.KQ_BF16,
                      cfg: N.kq_quant_cfg | None = None) -> int:
    out = ctypes.c_size_t(0)
    check(N.lib.kq_workspace_size(op, d_out, d_in, n_tok, dtype,
                                  ctypes.byref(cfg) if cfg is not None else None, ctypes.byref(out)))
    return out.value


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _ws(nbytes: int, device, ws, stream=None):
    """The caller's workspace, or a new one. A new one is freed when the
    binding returns, possibly with the call's kernels still queued: on a
    stream other than the current one it is recorded there, so the caching
    allocator does not hand it out again before that stream's work is done."""
    if ws is not None:
        return ws
    t = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)
    return t


def kq_accumulate_cov(X, Xq, G, alpha: float, beta: float, HX=None, D=None, HG=None,
                      ws=None, stream=None, want=("HX", "D", "HG")):
    """HX, D, HG <- alpha * (covariance of this chunk) + beta * old (see kq.h).

    X, Xq: (n_tok, d_in); G: (n_tok, d_out); uint16 (bf16 patterns) or float32.
    Outputs listed in ``want`` are allocated when not given.
    """
    ref = Xq if Xq is not None else G
    if ref is None:
        raise ValueError("Xq or G is required")
    if ref.dim() != 2 or ref.dtype not in (torch.float32, torch.uint16, torch.int16, torch.bfloat16):
        raise ValueError(f"inputs must be 2-D float32 or bf16 patterns, got {tuple(ref.shape)} {ref.dtype}")
    dt = N.KQ_F32 if ref.dtype == torch.float32 else N.KQ_BF16
    n_tok = ref.shape[0]
    d_in = Xq.shape[1] if Xq is not None else 8
    d_out = G.shape[1] if G is not None else 8
    f32 = torch.float32
    _expect(X, (n_tok, d_in), ref.dtype, "X")
    _expect(Xq, (n_tok, d_in), ref.dtype, "Xq")
    _expect(G, (n_tok, d_out), ref.dtype, "G")
    _expect(HX, (d_in, d_in), f32, "HX")
    _expect(D, (d_in, d_in), f32, "D")
    _expect(HG, (d_out, d_out), f32, "HG")
    _need_cuda(X, Xq, G, HX, D, HG, ws)
    dev = ref.device
    if HX is None and "HX" in want and Xq is not None:
        HX = torch.empty(d_in, d_in, dtype=torch.float32, device=dev)
    if D is None and "D" in want and X is not None and Xq is not None:
        D = torch.empty(d_in, d_in, dtype=torch.float32, device=dev)
    if HG is None and "HG" in want and G is not None:
        HG = torch.empty(d_out, d_out, dtype=torch.float32, device=dev)
    if ws is None:
        need = kq_workspace_size(N.KQ_OP_ACCUMULATE_COV, d_out, d_in, n_tok, dt)
        ws = _ws(need, dev, None, stream)
    check(N.lib.kq_accumulate_cov(_ptr(X), _ptr(Xq), _ptr(G), dt, n_tok, d_in, d_out, alpha, beta,
                                  _ptr(HX), _ptr(D), _ptr(HG), _ptr(ws), _nbytes(ws), _stream(stream)))
    return HX, D, HG


def kq_biip(W, HX, D, HG, sign_in, sign_out, blk_in: int = 0, blk_out: int = 0, s_x=None,
            s_g=None, ws=None, stream=None):
    """In-place bidirectional incoherence processing; returns (s_x, s_g)."""
    d_out, d_in = W.shape
    f32 = torch.float32
    _expect(W, (d_out, d_in), f32, "W")
    _expect(HX, (d_in, d_in), f32, "HX")
    _expect(D, (d_in, d_in), f32, "D")
    _expect(HG, (d_out, d_out), f32, "HG")
    _expect(sign_in, (d_in,), torch.int8, "sign_in")
    _expect(sign_out, (d_out,), torch.int8, "sign_out")
    _expect(s_x, (d_in,), f32, "s_x")
    _expect(s_g, (d_out,), f32, "s_g")
    _need_cuda(W, HX, D, HG, sign_in, sign_out, s_x, s_g, ws)
    dev = W.device
    if s_x is None:
        s_x = torch.empty(d_in, dtype=torch.float32, device=dev)
    if s_g is None:
        s_g = torch.empty(d_out, dtype=torch.float32, device=dev)
    ws = _ws(kq_workspace_size(N.KQ_OP_BIIP, d_out, d_in), dev, ws, stream)
    check(N.lib.kq_biip(_ptr(W), _ptr(HX), _ptr(D), _ptr(HG), d_out, d_in, _ptr(sign_in),
                        _ptr(sign_out), blk_in, blk_out, _ptr(s_x), _ptr(s_g), _ptr(ws), _nbytes(ws),
                        _stream(stream)))
    return s_x, s_g


def kq_sensitivity(HX, HG, ws=None, stream=None):
    """(tr HX, tr HG, s) as Python floats (synchronizes the stream)."""
    _expect(HX, (HX.shape[0], HX.shape[0]), torch.float32, "HX")
    _expect(HG, (HG.shape[0], HG.shape[0]), torch.float32, "HG")
    _need_cuda(HX, HG, ws)
    ws = _ws(kq_workspace_size(N.KQ_OP_SENSITIVITY, HG.shape[0], HX.shape[0]), HX.device, ws, stream)
    tx, tg, s = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    check(N.lib.kq_sensitivity(_ptr(HX), _ptr(HG), HX.shape[0], HG.shape[0], ctypes.byref(tx),
                               ctypes.byref(tg), ctypes.byref(s), _ptr(ws), _nbytes(ws),
                               _stream(stream)))
    return tx.value, tg.value, s.value


def kq_cholesky_inv(H, damp: float, U=None, ws=None, stream=None):
    """Upper U with U^T U = (H + damp*mean(diag H) I)^-1. Waits for the
    factorization (a non-positive pivot raises); the inverse is left queued
    on the stream."""
    n = H.shape[0]
    _expect(H, (n, n), torch.float32, "H")
    _expect(U, (n, n), torch.float32, "U")
    _need_cuda(H, U, ws)
    if U is None:
        U = torch.empty_like(H)
    ws = _ws(kq_workspace_size(N.KQ_OP_CHOLESKY_INV, n, n), H.device, ws, stream)
    info = ctypes.c_int32(0)
    st = N.lib.kq_cholesky_inv(_ptr(H), n, damp, _ptr(U), ctypes.byref(info), _ptr(ws), _nbytes(ws),
                               _stream(stream))
    check(st, info.value)
    return U


def kq_form_p(D, U, P=None, ws=None, stream=None):
    n = D.shape[0]
    for t, name in ((D, "D"), (U, "U"), (P, "P")):
        _expect(t, (n, n), torch.float32, name)
    _need_cuda(D, U, P, ws)
    if P is None:
        P = torch.empty_like(D)
    ws = _ws(kq_workspace_size(N.KQ_OP_FORM_P, n, n), D.device, ws, stream)
    check(N.lib.kq_form_p(_ptr(D), _ptr(U), n, _ptr(P), _ptr(ws), _nbytes(ws), _stream(stream)))
    return P


def kq_gptaq_quantize(W, U, D, bits: int, group: int = 0, block: int = 128, codes=None,
                      scale=None, zero=None, ws=None, stream=None):
    """In place W0' -> W^'; returns (codes, scale, zero)."""
    d_out, d_in = W.shape
    ng = -(-d_in // group) if group else 1
    f32 = torch.float32
    _expect(W, (d_out, d_in), f32, "W")
    _expect(U, (d_in, d_in), f32, "U")
    _expect(D, (d_in, d_in), f32, "D")
    _expect(codes, (d_out, d_in), torch.uint8, "codes")
    _expect(scale, (d_out, ng), f32, "scale")
    _expect(zero, (d_out, ng), f32, "zero")
    _need_cuda(W, U, D, codes, scale, zero, ws)
    dev = W.device
    cfg = N.kq_quant_cfg(bits, group, block, 0)
    if codes is None:
        codes = torch.empty(d_out, d_in, dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(d_out, ng, dtype=torch.float32, device=dev)
    if zero is None:
        zero = torch.empty(d_out, ng, dtype=torch.float32, device=dev)
    ws = _ws(kq_workspace_size(N.KQ_OP_GPTAQ_QUANTIZE, d_out, d_in, cfg=cfg), dev, ws, stream)
    check(N.lib.kq_gptaq_quantize(_ptr(W), _ptr(U), _ptr(D), d_out, d_in, ctypes.byref(cfg),
                                  _ptr(codes), _ptr(scale), _ptr(zero), _ptr(ws), _nbytes(ws),
                                  _stream(stream)))
    return codes, scale, zero


def kq_yaqa_quantize(W, U_in, U_out, D, bits: int, codes=None, scale=None, zero=None, ws=None,
                     stream=None):
    """In place W0' -> W^' with feedback along rows (U_in) and columns
    (U_out); returns (codes, scale, zero), one grid per output channel."""
    d_out, d_in = W.shape
    f32 = torch.float32
    _expect(W, (d_out, d_in), f32, "W")
    _expect(U_in, (d_in, d_in), f32, "U_in")
    _expect(U_out, (d_out, d_out), f32, "U_out")
    _expect(D, (d_in, d_in), f32, "D")
    _expect(codes, (d_out, d_in), torch.uint8, "codes")
    _expect(scale, (d_out, 1), f32, "scale")
    _expect(zero, (d_out, 1), f32, "zero")
    _need_cuda(W, U_in, U_out, D, codes, scale, zero, ws)
    dev = W.device
    cfg = N.kq_quant_cfg(bits, 0, 128, 0)
    if codes is None:
        codes = torch.empty(d_out, d_in, dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(d_out, 1, dtype=torch.float32, device=dev)
    if zero is None:
        zero = torch.empty(d_out, 1, dtype=torch.float32, device=dev)
    ws = _ws(kq_workspace_size(N.KQ_OP_YAQA_QUANTIZE, d_out, d_in, cfg=cfg), dev, ws, stream)
    check(N.lib.kq_yaqa_quantize(_ptr(W), _ptr(U_in), _ptr(U_out), _ptr(D), d_out, d_in,
                                 ctypes.byref(cfg), _ptr(codes), _ptr(scale), _ptr(zero), _ptr(ws),
                                 _nbytes(ws), _stream(stream)))
    return codes, scale, zero


def kq_allocate_bits(s, n_params, widths=(2, 3, 4), avg_budget: float = 2.5):
    L = len(s)
    sa = (ctypes.c_double * L)(*[float(v) for v in s])
    na = (ctypes.c_int64 * L)(*[int(v) for v in n_params])
    wa = (ctypes.c_int32 * len(widths))(*[int(v) for v in widths])
    out = (ctypes.c_int32 * L)()
    check(N.lib.kq_allocate_bits(sa, na, L, wa, len(widths), avg_budget, out))
    return [int(v) for v in out]


def kq_layer_objective(W0, What, HX, D, HG, ws=None, stream=None) -> float:
    d_out, d_in = W0.shape
    f32 = torch.float32
    _expect(W0, (d_out, d_in), f32, "W0")
    _expect(What, (d_out, d_in), f32, "What")
    _expect(HX, (d_in, d_in), f32, "HX")
    _expect(D, (d_in, d_in), f32, "D")
    _expect(HG, (d_out, d_out), f32, "HG")
    _need_cuda(W0, What, HX, D, HG, ws)
    ws = _ws(kq_workspace_size(N.KQ_OP_LAYER_OBJECTIVE, d_out, d_in), W0.device, ws, stream)
    obj = ctypes.c_double()
    check(N.lib.kq_layer_objective(_ptr(W0), _ptr(What), _ptr(HX), _ptr(D), _ptr(HG), d_out, d_in,
                                   ctypes.byref(obj), _ptr(ws), _nbytes(ws), _stream(stream)))
    return obj.value


def kq_set_kernel_events(op: int, start=None, stop=None, stream=None):
    """Bracket the main kernel of later `op` calls on this thread with two
    torch.cuda.Event objects (None, None switches the hook off). The events
    are recorded once here first so that their HIP handles exist."""
    if start is None and stop is None:
        check(N.lib.kq_set_kernel_events(op, None, None))
        return
    s = stream or torch.cuda.current_stream()
    for e in (start, stop):
        if not e.cuda_event:
            e.record(s)
    check(N.lib.kq_set_kernel_events(op, ctypes.c_void_p(start.cuda_event),
                                      ctypes.c_void_p(stop.cuda_event)))


def kq_set_gemm_tile(tile: int) -> None:
    """Force the fp32 product kernel of later calls on this thread: 0 chooses
    by shape (the default), 64, 128 or 256 force that fp32 tile where the
    product allows it, 3 the three-term bf16 kernel wherever it applies. A
    testing knob."""
    check(N.lib.kq_set_gemm_tile(int(tile)))


def kq_packed_row_words(d_in: int, bits: int) -> int:
    out = ctypes.c_int64(0)
    check(N.lib.kq_packed_row_words(d_in, bits, ctypes.byref(out)))
    return out.value


def kq_pack_codes(codes, bits: int, packed=None, stream=None):
    """uint8 codes (d_out x d_in) -> packed 32-bit words, stored as int32 (d_out x row words)."""
    d_out, d_in = codes.shape
    _expect(codes, (d_out, d_in), torch.uint8, "codes")
    if packed is not None:
        _expect(packed, (d_out, kq_packed_row_words(d_in, bits)), packed.dtype, "packed")
        if packed.element_size() != 4:
            raise ValueError("packed: expected 32-bit words")
    _need_cuda(codes, packed)
    if packed is None:
        packed = torch.empty(d_out, kq_packed_row_words(d_in, bits), dtype=torch.int32, device=codes.device)
    check(N.lib.kq_pack_codes(_ptr(codes), d_out, d_in, bits, _ptr(packed), _stream(stream)))
    return packed


def kq_apply_quantized(packed, bits: int, scale, zero, group: int, s_x, s_g, sign_in, sign_out, x,
                       blk_in: int = 0, blk_out: int = 0, y=None, ws=None, stream=None):
    """y = S_G^-1 U^T W^' V S_X^-1 x for x (batch x d_in fp32); returns y (batch x d_out)."""
    batch, d_in = x.shape
    d_out = packed.shape[0]
    f32 = torch.float32
    ng = -(-d_in // group) if group else 1
    _expect(x, (batch, d_in), f32, "x")
    _expect(packed, (d_out, kq_packed_row_words(d_in, bits)), packed.dtype, "packed")
    if packed.element_size() != 4:
        raise ValueError("packed: expected 32-bit words")
    _expect(scale, (d_out, ng), f32, "scale")
    _expect(zero, (d_out, ng), f32, "zero")
    _expect(s_x, (d_in,), f32, "s_x")
    _expect(s_g, (d_out,), f32, "s_g")
    _expect(sign_in, (d_in,), torch.int8, "sign_in")
    _expect(sign_out, (d_out,), torch.int8, "sign_out")
    _expect(y, (batch, d_out), f32, "y")
    _need_cuda(packed, scale, zero, s_x, s_g, sign_in, sign_out, x, y, ws)
    if y is None:
        y = torch.empty(batch, d_out, dtype=torch.float32, device=x.device)
    ws = _ws(kq_workspace_size(N.KQ_OP_APPLY_QUANTIZED, d_out, d_in, batch), x.device, ws, stream)
    check(N.lib.kq_apply_quantized(_ptr(packed), bits, _ptr(scale), _ptr(zero), group, _ptr(s_x),
                                   _ptr(s_g), _ptr(sign_in), _ptr(sign_out), blk_in, blk_out, _ptr(x),
                                   batch, d_out, d_in, _ptr(y), _ptr(ws), _nbytes(ws), _stream(stream)))
    return y


def kq_apply_quantized_noalloc(packed, bits: int, scale, zero, group: int, s_x, s_g, sign_in, sign_out,
                               x, y, blk_in: int = 0, blk_out: int = 0, stream=None):
    """kq_apply_quantized without a workspace: the library's fixed scratch
    array serves instead (for callers that cannot allocate). y (batch x
    d_out fp32) must be given: this call allocates nothing."""
    batch, d_in = x.shape
    d_out = packed.shape[0]
    f32 = torch.float32
    ng = -(-d_in // group) if group else 1
    if y is None:
        raise ValueError("y: expected an output tensor (this call allocates nothing)")
    _expect(x, (batch, d_in), f32, "x")
    _expect(packed, (d_out, kq_packed_row_words(d_in, bits)), packed.dtype, "packed")
    if packed.element_size() != 4:
        raise ValueError("packed: expected 32-bit words")
    _expect(scale, (d_out, ng), f32, "scale")
    _expect(zero, (d_out, ng), f32, "zero")
    _expect(s_x, (d_in,), f32, "s_x")
    _expect(s_g, (d_out,), f32, "s_g")
    _expect(sign_in, (d_in,), torch.int8, "sign_in")
    _expect(sign_out, (d_out,), torch.int8, "sign_out")
    _expect(y, (batch, d_out), f32, "y")
    _need_cuda(packed, scale, zero, s_x, s_g, sign_in, sign_out, x, y)
    check(N.lib.kq_apply_quantized_noalloc(_ptr(packed), bits, _ptr(scale), _ptr(zero), group, _ptr(s_x),
                                           _ptr(s_g), _ptr(sign_in), _ptr(sign_out), blk_in, blk_out,
                                           _ptr(x), batch, d_out, d_in, _ptr(y), _stream(stream)))
    return y


def kq_apply_quantized_a4(packed, scale, zero, s_x, s_g, sign_in, sign_out, x, clip: float = 1.0,
                          blk_in: int = 0, blk_out: int = 0, y=None, act_codes=None, act_scale=None,
                          ws=None, stream=None):
    """The product with 2-bit weights and 4-bit activations: x2 = V S_X^-1 x
    is rounded per vector to s * a (a in [-8, 7], s = clip * max|x2| / 7) and
    y = S_G^-1 U^T W^' (s a). Returns y (batch x d_out); act_codes (batch x
    d_in int8) and act_scale (batch fp32), if given, receive a and s."""
    batch, d_in = x.shape
    d_out = packed.shape[0]
    _expect(x, (batch, d_in), torch.float32, "x")
    _expect(packed, (d_out, kq_packed_row_words(d_in, 2)), packed.dtype, "packed")
    _expect(scale, (d_out,), torch.float32, "scale")
    _expect(zero, (d_out,), torch.float32, "zero")
    _expect(s_x, (d_in,), torch.float32, "s_x")
    _expect(s_g, (d_out,), torch.float32, "s_g")
    _expect(sign_in, (d_in,), torch.int8, "sign_in")
    _expect(sign_out, (d_out,), torch.int8, "sign_out")
    _expect(y, (batch, d_out), torch.float32, "y")
    _expect(act_codes, (batch, d_in), torch.int8, "act_codes")
    _expect(act_scale, (batch,), torch.float32, "act_scale")
    if packed.element_size() != 4:
        raise ValueError("packed: expected 32-bit words")
    _need_cuda(packed, scale, zero, s_x, s_g, sign_in, sign_out, x, y, act_codes, act_scale, ws)
    if y is None:
        y = torch.empty(batch, d_out, dtype=torch.float32, device=x.device)
    ws = _ws(kq_workspace_size(N.KQ_OP_APPLY_QUANTIZED_A4, d_out, d_in, batch), x.device, ws, stream)
    check(N.lib.kq_apply_quantized_a4(_ptr(packed), _ptr(scale), _ptr(zero), _ptr(s_x), _ptr(s_g),
                                      _ptr(sign_in), _ptr(sign_out), blk_in, blk_out, _ptr(x), batch,
                                      d_out, d_in, float(clip), _ptr(y), _ptr(act_codes),
                                      _ptr(act_scale), _ptr(ws), _nbytes(ws), _stream(stream)))
    return y
