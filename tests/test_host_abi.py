"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
validates arguments on the host before any launch, and its host-only
allocator matches the oracle. No compute call reaches a GPU here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from synth import layer_specs

kqn = pytest.importorskip("post_weight_quantization_amd._native")
N = kqn
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "kq.h")).read()
    declared = set(re.findall(r"^\s*(?:kq_status|const char\*)\s+(kq_\w+)\s*\(", hdr, re.M))
    assert declared == set(N.EXPORTS)
    for name in declared:
        assert hasattr(N.lib, name), name
    assert N.lib.kq_version().startswith(b"kq")


def _err(status):
    return status, N.lib.kq_last_error().decode()


def test_null_and_shape_validation():
    cfg = N.kq_quant_cfg(2, 0, 128, 0)
    st, msg = _err(N.lib.kq_gptaq_quantize(None, None, None, 4, 128, ctypes.byref(cfg), None, None,
                                           None, None, 0, None))
    assert st == N.KQ_ERR_ARG and "NULL" in msg
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    st, msg = _err(N.lib.kq_gptaq_quantize(fake, fake, None, 4, 100, ctypes.byref(cfg), fake, fake,
                                           fake, fake, 1 << 30, None))
    assert st == N.KQ_ERR_SHAPE and "128" in msg
    bad = N.kq_quant_cfg(2, 64, 128, 0)
    st, _ = _err(N.lib.kq_gptaq_quantize(fake, fake, None, 4, 128, ctypes.byref(bad), fake, fake,
                                         fake, fake, 1 << 30, None))
    assert st == N.KQ_ERR_UNSUPPORTED
    st, _ = _err(N.lib.kq_cholesky_inv(fake, 100, 0.01, ctypes.c_void_p(0x20000), None, fake, 1 << 30, None))
    assert st == N.KQ_ERR_SHAPE
    st, _ = _err(N.lib.kq_cholesky_inv(fake, 128, 0.01, fake, None, fake, 1 << 30, None))
    assert st == N.KQ_ERR_ARG  # aliasing
    st, _ = _err(N.lib.kq_cholesky_inv(fake, 128, float("nan"), ctypes.c_void_p(0x20000), None, fake,
                                       1 << 30, None))
    assert st == N.KQ_ERR_ARG
    st, msg = _err(N.lib.kq_biip(fake, fake, None, fake, 96, 128, fake, fake, 0, 48, None, None,
                                 fake, 1 << 30, None))
    assert st == N.KQ_ERR_SHAPE and "power of two" in msg
    st, _ = _err(N.lib.kq_biip(fake, fake, None, fake, 16384, 128, fake, fake, 0, 0, None, None,
                               fake, 1 << 30, None))
    assert st == N.KQ_ERR_UNSUPPORTED
    st, _ = _err(N.lib.kq_accumulate_cov(fake, fake, fake, 7, 64, 256, 256, 1.0, 0.0, fake, fake,
                                         fake, fake, 1 << 30, None))
    assert st == N.KQ_ERR_ARG
    st, _ = _err(N.lib.kq_accumulate_cov(None, fake, None, N.KQ_BF16, 64, 256, 256, 1.0, 0.0, None,
                                         fake, None, fake, 1 << 30, None))
    assert st == N.KQ_ERR_ARG  # D needs X
    st, _ = _err(N.lib.kq_accumulate_cov(fake, fake, fake, N.KQ_BF16, 64, 250, 256, 1.0, 0.0, fake,
                                         fake, fake, fake, 1 << 30, None))
    assert st == N.KQ_ERR_SHAPE


def test_kernel_event_hook_validation():
    fake = ctypes.c_void_p(0x10000)  # never recorded: the hook only stores it
    assert N.lib.kq_set_kernel_events(N.KQ_OP_BIIP, None, None) == N.KQ_ERR_UNSUPPORTED
    assert N.lib.kq_set_kernel_events(N.KQ_OP_ACCUMULATE_COV, fake, None) == N.KQ_ERR_ARG
    assert N.lib.kq_set_kernel_events(N.KQ_OP_ACCUMULATE_COV, None, None) == N.KQ_OK
    for op in (N.KQ_OP_GPTAQ_QUANTIZE, N.KQ_OP_APPLY_QUANTIZED, N.KQ_OP_APPLY_QUANTIZED_A4):
        assert N.lib.kq_set_kernel_events(op, None, None) == N.KQ_OK
    assert N.lib.kq_set_kernel_events(N.KQ_OP_YAQA_QUANTIZE, None, None) == N.KQ_ERR_UNSUPPORTED


def test_gemm_tile_knob_validation():
    for bad in (1, 2, 4, 32, 96, 512, -64):
        assert N.lib.kq_set_gemm_tile(bad) == N.KQ_ERR_ARG
    for ok in (3, 64, 128, 256, 0):
        assert N.lib.kq_set_gemm_tile(ok) == N.KQ_OK


def test_inference_entry_points_validate_on_host():
    from oracle import deploy
    out = ctypes.c_int64()
    for d_in, bits in ((4096, 2), (33, 3), (11008, 3), (1, 8)):
        assert N.lib.kq_packed_row_words(d_in, bits, ctypes.byref(out)) == N.KQ_OK
        assert out.value == deploy.packed_row_words(d_in, bits)
    assert N.lib.kq_packed_row_words(64, 5, ctypes.byref(out)) == N.KQ_ERR_ARG
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    args = lambda bits, group, d_out, d_in, ws: (fake, bits, fake, fake, group, fake, fake, fake, fake, 0,
                                                 0, fake, 1, d_out, d_in, fake, fake, ws, None)
    assert N.lib.kq_apply_quantized(*args(5, 0, 64, 64, 1 << 30)) == N.KQ_ERR_ARG
    assert N.lib.kq_apply_quantized(*args(2, 64, 64, 128, 1 << 30)) == N.KQ_ERR_UNSUPPORTED
    assert N.lib.kq_apply_quantized(*args(2, 0, 64, 48, 1 << 30)) == N.KQ_ERR_SHAPE
    assert N.lib.kq_apply_quantized(*args(2, 0, 6, 64, 1 << 30)) == N.KQ_ERR_SHAPE
    big = list(args(2, 0, 64, 64, 1 << 30))
    big[12] = 65537  # batch
    assert N.lib.kq_apply_quantized(*big) == N.KQ_ERR_SHAPE
    st = N.lib.kq_apply_quantized(*args(2, 0, 64, 64, 16))
    assert st == N.KQ_ERR_WORKSPACE
    assert N.lib.kq_pack_codes(None, 4, 4, 2, fake, None) == N.KQ_ERR_ARG


def test_workspace_checked_before_launch():
    fake = ctypes.c_void_p(0x10000)
    cfg = N.kq_quant_cfg(2, 0, 128, 0)
    need = ctypes.c_size_t()
    assert N.lib.kq_workspace_size(N.KQ_OP_GPTAQ_QUANTIZE, 256, 512, 0, 0, ctypes.byref(cfg),
                                   ctypes.byref(need)) == 0
    assert need.value >= 256 * 512 * 4 + 2 * 512 * 512 * 4
    st, msg = _err(N.lib.kq_gptaq_quantize(fake, fake, fake, 256, 512, ctypes.byref(cfg), fake, fake,
                                           fake, fake, need.value - 1, None))
    assert st == N.KQ_ERR_WORKSPACE and str(need.value) in msg
    for op in range(8):
        assert N.lib.kq_workspace_size(op, 1024, 4096, 8192, 0, ctypes.byref(cfg), ctypes.byref(need)) == 0
    assert N.lib.kq_workspace_size(99, 1, 1, 1, 0, None, ctypes.byref(need)) == N.KQ_ERR_ARG


def test_allocate_bits_matches_oracle():
    api = pytest.importorskip("post_weight_quantization_amd.api")
    rng = np.random.default_rng(0)
    n = [sp.n_params for sp in layer_specs(4)]
    for trial in range(200):
        s = list(rng.lognormal(0, 2, 7))
        if trial % 7 == 0:
            s[3] = s[0]
        avg = float(rng.uniform(2.0, 4.0))
        assert api.kq_allocate_bits(s, n, (2, 3, 4), avg) == oracle.allocate_bits(s, n, (2, 3, 4), avg)
    with pytest.raises(N.KQError):
        api.kq_allocate_bits([1.0], [10], (2, 3, 4), 1.5)


def test_yaqa_validation():
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    cfg = N.kq_quant_cfg(2, 0, 128, 0)
    st, msg = _err(N.lib.kq_yaqa_quantize(None, fake, fake, None, 4, 64, ctypes.byref(cfg), fake,
                                          fake, fake, fake, 1 << 30, None))
    assert st == N.KQ_ERR_ARG and "NULL" in msg
    st, msg = _err(N.lib.kq_yaqa_quantize(fake, fake, fake, None, 0, 64, ctypes.byref(cfg), fake,
                                          fake, fake, fake, 1 << 30, None))
    assert st == N.KQ_ERR_SHAPE
    grouped = N.kq_quant_cfg(2, 128, 128, 0)
    st, msg = _err(N.lib.kq_yaqa_quantize(fake, fake, fake, None, 4, 128, ctypes.byref(grouped), fake,
                                          fake, fake, fake, 1 << 30, None))
    assert st == N.KQ_ERR_UNSUPPORTED and "group" in msg
    need = ctypes.c_size_t()
    assert N.lib.kq_workspace_size(N.KQ_OP_YAQA_QUANTIZE, 100, 200, 0, 0, ctypes.byref(cfg),
                                   ctypes.byref(need)) == 0
    # three padded 128 x 256 work matrices, padded U_in and U_out, padded D, P and T
    assert need.value >= 4 * (3 * 128 * 256 + 3 * 256 * 256 + 128 * 128)
    st, msg = _err(N.lib.kq_yaqa_quantize(fake, fake, fake, fake, 100, 200, ctypes.byref(cfg), fake,
                                          fake, fake, fake, need.value - 1, None))
    assert st == N.KQ_ERR_WORKSPACE


def test_apply_a4_validation():
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    f = N.lib.kq_apply_quantized_a4

    def call(packed=fake, x=fake, batch=2, d_out=64, d_in=1024, clip=1.0, codes=None, ws_bytes=1 << 30,
             blk_in=0):
        return _err(f(packed, fake, fake, fake, fake, fake, fake, blk_in, 0, x, batch, d_out, d_in, clip,
                      fake, codes, None, fake, ws_bytes, None))

    st, msg = call(packed=None)
    assert st == N.KQ_ERR_ARG and "NULL" in msg
    for clip in (0.0, -0.5, 1.5, float("nan")):
        st, msg = call(clip=clip)
        assert st == N.KQ_ERR_ARG and "clip" in msg
    st, _ = call(d_in=1000)
    assert st == N.KQ_ERR_SHAPE
    st, _ = call(d_out=66)
    assert st == N.KQ_ERR_SHAPE
    st, _ = call(batch=0)
    assert st == N.KQ_ERR_SHAPE
    st, msg = call(batch=65537)
    assert st == N.KQ_ERR_SHAPE and "65536" in msg
    st, _ = call(blk_in=3)
    assert st == N.KQ_ERR_SHAPE
    st, msg = call(codes=ctypes.c_void_p(0x10004))
    assert st == N.KQ_ERR_ARG and "aligned" in msg
    need = ctypes.c_size_t()
    assert N.lib.kq_workspace_size(N.KQ_OP_APPLY_QUANTIZED_A4, 64, 1024, 20, 0, None,
                                   ctypes.byref(need)) == 0
    # x2 and y1 in fp32, one byte per input value in two 16-vector tiles
    assert need.value >= 4 * 20 * 1024 + 4 * 20 * 64 + 32 * 1024
    st, _ = call(batch=20, ws_bytes=need.value - 1)
    assert st == N.KQ_ERR_WORKSPACE


def test_bindings_reject_wrong_shapes_before_any_launch():
    """Every binding checks the shape and dtype of each tensor it hands to the
    library as a raw pointer; a wrong one raises ValueError on the host (these
    CPU tensors would otherwise be rejected only for not being on the GPU)."""
    import torch

    from post_weight_quantization_amd import api

    f32, i8, u8 = torch.float32, torch.int8, torch.uint8
    z = lambda *s, dt=f32: torch.zeros(*s, dtype=dt)
    cases = [
        ("HX", lambda: api.kq_accumulate_cov(z(64, 256), z(64, 256), z(64, 128), 1.0, 0.0,
                                             HX=z(255, 256))),
        ("G", lambda: api.kq_accumulate_cov(z(64, 256), z(64, 256), z(63, 128), 1.0, 0.0)),
        ("HG", lambda: api.kq_biip(z(128, 256), z(256, 256), None, z(128, 127), z(256, dt=i8),
                                   z(128, dt=i8))),
        ("sign_in", lambda: api.kq_biip(z(128, 256), z(256, 256), None, z(128, 128), z(256, dt=f32),
                                        z(128, dt=i8))),
        ("U", lambda: api.kq_cholesky_inv(z(256, 256), 0.01, U=z(128, 256))),
        ("P", lambda: api.kq_form_p(z(256, 256), z(256, 256), P=z(256, 255))),
        ("scale", lambda: api.kq_gptaq_quantize(z(64, 256), z(256, 256), None, 3, 128,
                                                scale=z(64, 1), zero=z(64, 2))),
        ("codes", lambda: api.kq_gptaq_quantize(z(64, 256), z(256, 256), None, 2,
                                                codes=z(64, 256, dt=f32))),
        ("D", lambda: api.kq_gptaq_quantize(z(64, 256), z(256, 256), z(64, 256), 2)),
        ("HG", lambda: api.kq_layer_objective(z(64, 256), z(64, 256), z(256, 256), None, z(256, 256))),
        ("U_out", lambda: api.kq_yaqa_quantize(z(64, 256), z(256, 256), z(256, 256), None, 2)),
        ("packed", lambda: api.kq_apply_quantized(z(64, 4, dt=torch.int32), 2, z(64, 1), z(64, 1), 0,
                                                  z(256), z(64), z(256, dt=i8), z(64, dt=i8),
                                                  z(2, 256))),
        ("scale", lambda: api.kq_apply_quantized(z(64, 24, dt=torch.int32), 3, z(64, 1), z(64, 1), 128,
                                                 z(256), z(64), z(256, dt=i8), z(64, dt=i8),
                                                 z(2, 256))),
        ("packed", lambda: api.kq_pack_codes(z(64, 256, dt=u8), 2, packed=z(64, 15, dt=torch.int32))),
        ("x", lambda: api.kq_apply_quantized_a4(z(64, 32, dt=torch.int32), z(64), z(64), z(512), z(64),
                                                z(512, dt=i8), z(64, dt=i8), z(2, 512, dt=torch.float64))),
    ]
    for name, call in cases:
        with pytest.raises(ValueError, match=rf"^{name}: expected"):
            call()
