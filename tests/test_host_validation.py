"""Every argument check of the C ABI, one case each (CPU).

Each case passes the checks before the one it targets and fails that one, so
a check that is removed or weakened lets its case through to the next check
(or to a launch) and fails here. The device pointers are fake addresses that
no code path reaches: every case must be rejected on the host, before any
launch, with the status the header documents for it.
"""
import ctypes
import math

import pytest

N = pytest.importorskip("post_weight_quantization_amd._native")


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


# a fake device pointer must never reach a launch on a real device
pytestmark = pytest.mark.skipif(_gpu_present(), reason="fake device pointers: host-only checks")

A = ctypes.c_void_p(0x100000)      # 16-byte aligned stand-ins for device buffers
B = ctypes.c_void_p(0x200000)
C = ctypes.c_void_p(0x300000)
MIS = ctypes.c_void_p(0x100004)    # misaligned
BIG = 1 << 40                      # a workspace size that passes every size check
ARG, SHAPE, WS, UNS, NONFIN = (N.KQ_ERR_ARG, N.KQ_ERR_SHAPE, N.KQ_ERR_WORKSPACE,
                               N.KQ_ERR_UNSUPPORTED, N.KQ_ERR_NONFINITE)


def cfg(bits=2, group=0, block=128, flags=0):
    return ctypes.byref(N.kq_quant_cfg(bits, group, block, flags))


def cov(X=A, Xq=A, G=A, dt=N.KQ_BF16, n=64, d_in=256, d_out=256, alpha=1.0, beta=0.0, HX=B, D=B,
        HG=B, ws=C, wsb=BIG):
    return N.lib.kq_accumulate_cov(X, Xq, G, dt, n, d_in, d_out, alpha, beta, HX, D, HG, ws, wsb, None)


def biip(W=A, HX=A, D=None, HG=A, d_out=256, d_in=256, si=B, so=B, bi=0, bo=0, ws=C, wsb=BIG):
    return N.lib.kq_biip(W, HX, D, HG, d_out, d_in, si, so, bi, bo, None, None, ws, wsb, None)


def sens(HX=A, HG=A, d_in=256, d_out=256, ws=C, wsb=BIG):
    return N.lib.kq_sensitivity(HX, HG, d_in, d_out, None, None, None, ws, wsb, None)


def chol(H=A, n=256, damp=0.01, U=B, ws=C, wsb=BIG):
    return N.lib.kq_cholesky_inv(H, n, damp, U, None, ws, wsb, None)


def formp(D=A, U=B, n=256, P=C, ws=C, wsb=BIG):
    return N.lib.kq_form_p(D, U, n, P, ws, wsb, None)


def gptaq(W=A, U=B, D=None, d_out=64, d_in=256, c=None, codes=C, scale=C, zero=C, ws=C, wsb=BIG):
    return N.lib.kq_gptaq_quantize(W, U, D, d_out, d_in, c if c is not None else cfg(), codes, scale,
                                   zero, ws, wsb, None)


def yaqa(W=A, Ui=B, Uo=B, D=None, d_out=64, d_in=256, c=None, codes=C, scale=C, zero=C, ws=C, wsb=BIG):
    return N.lib.kq_yaqa_quantize(W, Ui, Uo, D, d_out, d_in, c if c is not None else cfg(), codes,
                                  scale, zero, ws, wsb, None)


def obj(W0=A, Wh=A, HX=A, D=None, HG=A, d_out=64, d_in=64, out=True, ws=C, wsb=BIG):
    o = ctypes.c_double()
    return N.lib.kq_layer_objective(W0, Wh, HX, D, HG, d_out, d_in, ctypes.byref(o) if out else None,
                                    ws, wsb, None)


def apply(packed=A, bits=2, scale=B, zero=B, group=0, s_x=A, s_g=B, si=B, so=B, bi=0, bo=0, x=A,
          batch=1, d_out=64, d_in=64, y=A, ws=C, wsb=BIG):
    return N.lib.kq_apply_quantized(packed, bits, scale, zero, group, s_x, s_g, si, so, bi, bo, x, batch,
                                    d_out, d_in, y, ws, wsb, None)


def apply_na(packed=A, bits=2, d_out=64, d_in=64, batch=1, y=A):
    return N.lib.kq_apply_quantized_noalloc(packed, bits, B, B, 0, A, B, B, B, 0, 0, A, batch, d_out, d_in,
                                            y, None)


def a4(packed=A, scale=B, zero=B, s_x=A, s_g=B, si=B, so=B, bi=0, bo=0, x=A, batch=1, d_out=64,
       d_in=512, clip=1.0, y=A, codes=None, ws=C, wsb=BIG):
    return N.lib.kq_apply_quantized_a4(packed, scale, zero, s_x, s_g, si, so, bi, bo, x, batch, d_out,
                                       d_in, clip, y, codes, None, ws, wsb, None)


def alloc(s=(1.0, 2.0), n=(10, 10), widths=(2, 3, 4), budget=2.5, null=False):
    L, W = len(s), len(widths)
    sa = (ctypes.c_double * max(L, 1))(*s)
    na = (ctypes.c_int64 * max(L, 1))(*n)
    wa = (ctypes.c_int32 * max(W, 1))(*widths)
    out = (ctypes.c_int32 * max(L, 1))()
    return N.lib.kq_allocate_bits(None if null else sa, na, L, wa, W, budget, out)


def wsize(op, d_out=64, d_in=64, n_tok=64, dtype=N.KQ_BF16, out=True):
    b = ctypes.c_size_t()
    return N.lib.kq_workspace_size(op, d_out, d_in, n_tok, dtype, None, ctypes.byref(b) if out else None)


CASES = [
    # accumulate_cov
    ("cov bad dtype", lambda: cov(dt=7), ARG, "dtype"),
    ("cov no output", lambda: cov(HX=None, D=None, HG=None), ARG, "no output"),
    ("cov HX without Xq", lambda: cov(Xq=None, D=None, HG=None), ARG, "need Xq"),
    ("cov D without X", lambda: cov(X=None), ARG, "D needs X"),
    ("cov HG without G", lambda: cov(G=None), ARG, "HG needs G"),
    ("cov no tokens", lambda: cov(n=0), SHAPE, ">= 1"),
    ("cov d_in zero", lambda: cov(d_in=0), SHAPE, ">= 1"),
    ("cov d_out zero", lambda: cov(d_out=0), SHAPE, ">= 1"),
    ("cov d_in not /8", lambda: cov(d_in=252), SHAPE, "multiples of 8"),
    ("cov d_out not /8", lambda: cov(d_out=260), SHAPE, "multiples of 8"),
    ("cov fp32 ragged tokens", lambda: cov(dt=N.KQ_F32, n=62), SHAPE, "multiple of 4"),
    ("cov alpha nan", lambda: cov(alpha=math.nan), ARG, "finite"),
    ("cov beta inf", lambda: cov(beta=math.inf), ARG, "finite"),
    ("cov misaligned input", lambda: cov(Xq=MIS), ARG, "aligned"),
    ("cov misaligned output", lambda: cov(HG=MIS), ARG, "aligned"),
    ("cov no workspace", lambda: cov(ws=None), WS, "NULL"),
    ("cov small workspace", lambda: cov(wsb=64), WS, "required"),
    ("cov misaligned workspace", lambda: cov(ws=MIS), ARG, "workspace must be 16-byte aligned"),
    # biip
    ("biip null W", lambda: biip(W=None), ARG, "NULL"),
    ("biip null sign", lambda: biip(so=None), ARG, "NULL"),
    ("biip d_in not /4", lambda: biip(d_in=254), SHAPE, "multiples of 4"),
    ("biip d_out tiny", lambda: biip(d_out=0), SHAPE, "multiples of 4"),
    ("biip misaligned D", lambda: biip(D=MIS), ARG, "aligned"),
    ("biip block not a power of two", lambda: biip(bi=48), SHAPE, "power of two"),
    ("biip block not dividing", lambda: biip(d_in=96, bi=64), SHAPE, "dividing"),
    ("biip negative block", lambda: biip(bo=-2), SHAPE, "power of two"),
    ("biip block above 8192", lambda: biip(d_out=16384), UNS, "8192"),
    ("biip small workspace", lambda: biip(wsb=16), WS, "required"),
    # sensitivity
    ("sens null", lambda: sens(HG=None), ARG, "NULL"),
    ("sens size zero", lambda: sens(d_out=0), SHAPE, ">= 1"),
    ("sens no workspace", lambda: sens(ws=None), WS, "NULL"),
    # cholesky_inv
    ("chol null", lambda: chol(U=None), ARG, "NULL"),
    ("chol aliasing", lambda: chol(U=A), ARG, "distinct"),
    ("chol n not /128", lambda: chol(n=200), SHAPE, "multiple of 128"),
    ("chol n zero", lambda: chol(n=0), SHAPE, "multiple of 128"),
    ("chol damp negative", lambda: chol(damp=-0.01), ARG, "damp"),
    ("chol damp nan", lambda: chol(damp=math.nan), ARG, "damp"),
    ("chol misaligned", lambda: chol(H=MIS), ARG, "aligned"),
    ("chol small workspace", lambda: chol(wsb=1024), WS, "required"),
    # form_p
    ("formp null", lambda: formp(D=None), ARG, "NULL"),
    ("formp P aliases U", lambda: formp(P=B), ARG, "alias"),
    ("formp P aliases D", lambda: formp(P=A), ARG, "alias"),
    ("formp n not /128", lambda: formp(n=130), SHAPE, "multiple of 128"),
    ("formp misaligned", lambda: formp(U=MIS), ARG, "aligned"),
    ("formp small workspace", lambda: formp(ws=ctypes.c_void_p(0x400000), wsb=1024), WS, "required"),
    # gptaq_quantize
    ("gptaq null", lambda: gptaq(codes=None), ARG, "NULL"),
    ("gptaq d_out zero", lambda: gptaq(d_out=0), SHAPE, "d_out"),
    ("gptaq cfg null", lambda: gptaq(c=ctypes.POINTER(N.kq_quant_cfg)()), ARG, "cfg"),
    ("gptaq bits 0", lambda: gptaq(c=cfg(bits=0)), ARG, "bits"),
    ("gptaq bits 9", lambda: gptaq(c=cfg(bits=9)), ARG, "bits"),
    ("gptaq group 64", lambda: gptaq(c=cfg(group=64)), UNS, "group"),
    ("gptaq block 64", lambda: gptaq(c=cfg(block=64)), UNS, "block"),
    ("gptaq flags", lambda: gptaq(c=cfg(flags=1)), ARG, "flags"),
    ("gptaq d_in not /128", lambda: gptaq(d_in=200), SHAPE, "multiple of 128"),
    ("gptaq d_in zero", lambda: gptaq(d_in=0), SHAPE, "multiple of 128"),
    ("gptaq d_in negative", lambda: gptaq(d_in=-128), SHAPE, "multiple of 128"),
    ("gptaq misaligned", lambda: gptaq(W=MIS), ARG, "aligned"),
    ("gptaq small workspace", lambda: gptaq(wsb=64), WS, "required"),
    # yaqa_quantize
    ("yaqa null", lambda: yaqa(Uo=None), ARG, "NULL"),
    ("yaqa size zero", lambda: yaqa(d_in=0), SHAPE, ">= 1"),
    ("yaqa cfg null", lambda: yaqa(c=ctypes.POINTER(N.kq_quant_cfg)()), ARG, "cfg"),
    ("yaqa bits 9", lambda: yaqa(c=cfg(bits=9)), ARG, "bits"),
    ("yaqa group", lambda: yaqa(c=cfg(group=128)), UNS, "group"),
    ("yaqa block", lambda: yaqa(c=cfg(block=256)), UNS, "block"),
    ("yaqa flags", lambda: yaqa(c=cfg(flags=2)), ARG, "flags"),
    ("yaqa huge", lambda: yaqa(d_in=(1 << 24) + 128), SHAPE, "2^24"),
    ("yaqa misaligned", lambda: yaqa(D=MIS), ARG, "aligned"),
    ("yaqa small workspace", lambda: yaqa(wsb=64), WS, "required"),
    # layer_objective
    ("objective null out", lambda: obj(out=False), ARG, "NULL"),
    ("objective null HG", lambda: obj(HG=None), ARG, "NULL"),
    ("objective d_in not /4", lambda: obj(d_in=62), SHAPE, "multiples of 4"),
    ("objective misaligned", lambda: obj(Wh=MIS), ARG, "aligned"),
    ("objective small workspace", lambda: obj(wsb=8), WS, "required"),
    # packing
    ("row words null", lambda: N.lib.kq_packed_row_words(64, 2, None), ARG, "NULL"),
    ("row words bits 5", lambda: N.lib.kq_packed_row_words(64, 5, ctypes.byref(ctypes.c_int64())), ARG,
     "bits"),
    ("row words d_in 0", lambda: N.lib.kq_packed_row_words(0, 2, ctypes.byref(ctypes.c_int64())), SHAPE,
     ">= 1"),
    ("pack null", lambda: N.lib.kq_pack_codes(None, 4, 4, 2, A, None), ARG, "NULL"),
    ("pack bits 1", lambda: N.lib.kq_pack_codes(A, 4, 4, 1, B, None), ARG, "bits"),
    ("pack size 0", lambda: N.lib.kq_pack_codes(A, 0, 4, 2, B, None), SHAPE, "sizes"),
    ("pack misaligned", lambda: N.lib.kq_pack_codes(A, 4, 4, 2, MIS, None), ARG, "aligned"),
    # apply_quantized (and its no-allocation variant, which shares the checks)
    ("apply null", lambda: apply(zero=None), ARG, "NULL"),
    ("apply bits 5", lambda: apply(bits=5), ARG, "bits"),
    ("apply group 32", lambda: apply(group=32), UNS, "group"),
    ("apply d_out not /4", lambda: apply(d_out=66), SHAPE, "d_out"),
    ("apply batch 0", lambda: apply(batch=0), SHAPE, "batch"),
    ("apply batch too large", lambda: apply(batch=65537), SHAPE, "batch"),
    ("apply d_in not /32", lambda: apply(d_in=48), SHAPE, "multiple of 32"),
    ("apply d_in not /group", lambda: apply(group=128, d_in=96), SHAPE, "multiple of 32"),
    ("apply block", lambda: apply(bi=24), SHAPE, "power of two"),
    ("apply misaligned", lambda: apply(y=MIS), ARG, "aligned"),
    ("apply small workspace", lambda: apply(wsb=4), WS, "required"),
    ("noalloc bits", lambda: apply_na(bits=7), ARG, "bits"),
    ("noalloc misaligned", lambda: apply_na(packed=MIS), ARG, "aligned"),
    ("noalloc above the scratch size", lambda: apply_na(d_out=4096, d_in=4096, batch=65536), WS,
     "scratch"),
    # apply_quantized_a4
    ("a4 null", lambda: a4(x=None), ARG, "NULL"),
    ("a4 clip 0", lambda: a4(clip=0.0), ARG, "clip"),
    ("a4 clip above 1", lambda: a4(clip=1.5), ARG, "clip"),
    ("a4 clip nan", lambda: a4(clip=math.nan), ARG, "clip"),
    ("a4 d_out not /4", lambda: a4(d_out=10), SHAPE, "d_out"),
    ("a4 batch 0", lambda: a4(batch=0), SHAPE, "batch"),
    ("a4 d_in not /512", lambda: a4(d_in=768), SHAPE, "512"),
    ("a4 d_in above 2^24", lambda: a4(d_in=(1 << 24) + 512), SHAPE, "2^24"),
    ("a4 block", lambda: a4(bo=3), SHAPE, "power of two"),
    ("a4 misaligned codes", lambda: a4(codes=MIS), ARG, "aligned"),
    ("a4 small workspace", lambda: a4(wsb=4), WS, "required"),
    # allocate_bits (host only)
    ("alloc null", lambda: alloc(null=True), ARG, "NULL"),
    ("alloc no sublayers", lambda: alloc(s=(), n=()), ARG, ">= 1"),
    ("alloc no widths", lambda: alloc(widths=()), ARG, ">= 1"),
    ("alloc budget nan", lambda: alloc(budget=math.nan), ARG, "finite"),
    ("alloc repeated width", lambda: alloc(widths=(2, 2, 4)), ARG, "distinct"),
    ("alloc zero width", lambda: alloc(widths=(0, 2)), ARG, "distinct"),
    ("alloc negative count", lambda: alloc(n=(10, -1)), ARG, "negative"),
    ("alloc non-finite s", lambda: alloc(s=(1.0, math.inf)), NONFIN, "sensitivity"),
    ("alloc budget too small", lambda: alloc(budget=1.5), ARG, "below"),
    # workspace_size
    ("wsize null", lambda: wsize(N.KQ_OP_BIIP, out=False), ARG, "NULL"),
    ("wsize d_in 0", lambda: wsize(N.KQ_OP_BIIP, d_in=0), SHAPE, "d_in"),
    ("wsize cov tokens", lambda: wsize(N.KQ_OP_ACCUMULATE_COV, n_tok=0), SHAPE, "sizes"),
    ("wsize cov dtype", lambda: wsize(N.KQ_OP_ACCUMULATE_COV, dtype=5), ARG, "dtype"),
    ("wsize biip d_out", lambda: wsize(N.KQ_OP_BIIP, d_out=0), SHAPE, "sizes"),
    ("wsize gptaq d_out", lambda: wsize(N.KQ_OP_GPTAQ_QUANTIZE, d_out=0), SHAPE, "sizes"),
    ("wsize objective d_out", lambda: wsize(N.KQ_OP_LAYER_OBJECTIVE, d_out=0), SHAPE, "sizes"),
    ("wsize apply batch", lambda: wsize(N.KQ_OP_APPLY_QUANTIZED, n_tok=0), SHAPE, "sizes"),
    ("wsize yaqa d_out", lambda: wsize(N.KQ_OP_YAQA_QUANTIZE, d_out=0), SHAPE, "sizes"),
    ("wsize a4 batch", lambda: wsize(N.KQ_OP_APPLY_QUANTIZED_A4, n_tok=0), SHAPE, "sizes"),
    ("wsize unknown op", lambda: wsize(42), ARG, "unknown op"),
    # knobs
    ("gemm tile 32", lambda: N.lib.kq_set_gemm_tile(32), ARG, "tile"),
    ("events on an untimed op", lambda: N.lib.kq_set_kernel_events(N.KQ_OP_FORM_P, None, None), UNS,
     "timed kernel"),
    ("events half given", lambda: N.lib.kq_set_kernel_events(N.KQ_OP_ACCUMULATE_COV, None, A), ARG,
     "both"),
]


@pytest.mark.parametrize("name,call,status,words", CASES, ids=[c[0] for c in CASES])
def test_rejected_on_the_host(name, call, status, words):
    st = call()
    msg = N.lib.kq_last_error().decode()
    assert N.STATUS_NAMES.get(st) == N.STATUS_NAMES[status], (name, st, msg)
    assert words in msg, (name, msg)


def test_the_table_reaches_every_check_of_the_abi_source():
    """Every failure message in kq_api.hip that a host call can reach is
    produced by some case of the table."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(N.__file__), "csrc", "kq_api.hip")).read()
    msgs = set(re.findall(r'fail\(KQ_ERR_\w+,\s*"([^"]+)"', src))
    # reached only with a device present or from inside the library
    device_only = {m for m in msgs if m.startswith(("apply_quantized_noalloc: device index",
                                                    "apply_quantized_noalloc: no device address",
                                                    "internal read-back", "sensitivity: non-finite"))}
    reached = set()
    for _, call, _, _ in CASES:
        call()
        reached.add(N.lib.kq_last_error().decode())
    missing = []
    for m in sorted(msgs - device_only):
        # printf fields match anything; a message split over several string
        # literals is matched on its first one
        pat = re.escape(re.sub(r"%(?:zu|lld|d|s)", "\x00", m)).replace("\x00", ".*")
        if not any(re.match(pat, r) for r in reached):
            missing.append(m)
    assert not missing, missing


def _need(op, d_out, d_in, n_tok=64, c=None):
    b = ctypes.c_size_t()
    assert N.lib.kq_workspace_size(op, d_out, d_in, n_tok, N.KQ_BF16, c, ctypes.byref(b)) == N.KQ_OK
    return b.value


WS_EDGE = [
    ("cov", N.KQ_OP_ACCUMULATE_COV, lambda w: cov(wsb=w)),
    ("biip", N.KQ_OP_BIIP, lambda w: biip(wsb=w)),
    ("chol", N.KQ_OP_CHOLESKY_INV, lambda w: chol(wsb=w)),
    ("formp", N.KQ_OP_FORM_P, lambda w: formp(ws=ctypes.c_void_p(0x400000), wsb=w)),
    # the reported size covers the drift term, so these pass D
    ("gptaq", N.KQ_OP_GPTAQ_QUANTIZE, lambda w: gptaq(D=C, wsb=w)),
    ("yaqa", N.KQ_OP_YAQA_QUANTIZE, lambda w: yaqa(D=C, wsb=w)),
    ("objective", N.KQ_OP_LAYER_OBJECTIVE, lambda w: obj(wsb=w)),
    ("apply", N.KQ_OP_APPLY_QUANTIZED, lambda w: apply(wsb=w)),
    ("a4", N.KQ_OP_APPLY_QUANTIZED_A4, lambda w: a4(wsb=w)),
]
SHAPES = {"cov": (256, 256, 64), "biip": (256, 256), "chol": (64, 256), "formp": (64, 256),
          "gptaq": (64, 256), "yaqa": (64, 256), "objective": (64, 64), "apply": (64, 64, 1),
          "a4": (64, 512, 1)}


@pytest.mark.parametrize("name,op,call", WS_EDGE, ids=[w[0] for w in WS_EDGE])
def test_workspace_one_byte_short(name, op, call):
    """The size that kq_workspace_size reports is the exact minimum each call
    accepts for the same sizes: one byte less is rejected (the call with the
    full size would launch, so it is left to the GPU tests)."""
    need = _need(op, *SHAPES[name])
    assert need > 0
    st = call(need - 1)
    msg = N.lib.kq_last_error().decode()
    assert st == N.KQ_ERR_WORKSPACE and str(need) in msg, (name, need, msg)
