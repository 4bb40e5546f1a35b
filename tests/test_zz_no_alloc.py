"""The no-allocation inference entry point (kq_apply_quantized_noalloc)
against kq_apply_quantized on the same inputs: two calls in a row on the
library's fixed scratch array, the second with a smaller batch (and other
data), each bit-identical to the entry point with a caller workspace (the
same kernels run on the same values), on the matrix-core path (2-bit, one
grid per row) and the generic path (3-bit, groups of 128)."""
import numpy as np
import pytest

from tests.gpu_util import dev, have_gpu, host

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

if have_gpu():
    import torch

    import post_weight_quantization_amd as kq
    from post_weight_quantization_amd import _native as N


def _layer(rng, d_out, d_in, bits, group):
    ng = d_in // group if group else 1
    codes = rng.integers(0, 1 << bits, (d_out, d_in)).astype(np.uint8)
    return dict(packed=kq.kq_pack_codes(dev(codes), bits),
                scale=dev(rng.uniform(0.005, 0.02, (d_out, ng)).astype(np.float32)),
                zero=dev(rng.integers(0, 1 << bits, (d_out, ng)).astype(np.float32)),
                s_x=dev(np.exp(rng.normal(0, 0.5, d_in)).astype(np.float32)),
                s_g=dev(np.exp(rng.normal(0, 0.5, d_out)).astype(np.float32)),
                sign_in=dev(rng.choice([-1, 1], d_in).astype(np.int8)),
                sign_out=dev(rng.choice([-1, 1], d_out).astype(np.int8)))


@pytest.mark.parametrize("d_out,d_in,bits,group", [(1024, 4096, 2, 0), (512, 1536, 3, 128)])
def test_noalloc_matches_workspace_entry_point(d_out, d_in, bits, group):
    rng = np.random.default_rng(d_in + bits)
    L = _layer(rng, d_out, d_in, bits, group)
    args = (L["packed"], bits, L["scale"], L["zero"], group, L["s_x"], L["s_g"], L["sign_in"],
            L["sign_out"])
    for batch in (9, 3):
        print(f"[no-alloc] {d_out}x{d_in} {bits}-bit group {group} batch {batch}", flush=True)
        x = dev(rng.standard_normal((batch, d_in)).astype(np.float32))
        y_ref = kq.kq_apply_quantized(*args, x)
        y = torch.full((batch, d_out), float("nan"), dtype=torch.float32, device="cuda")
        kq.kq_apply_quantized_noalloc(*args, x, y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), host(y_ref))


def test_noalloc_rejects_sizes_beyond_the_scratch():
    d_out, d_in, batch = 8192, 28672, 4096
    need = kq.kq_workspace_size(N.KQ_OP_APPLY_QUANTIZED, d_out, d_in, batch)
    assert need > N.KQ_NOALLOC_SCRATCH_BYTES
    rng = np.random.default_rng(5)
    L = _layer(rng, 64, 512, 2, 0)  # small real buffers: validation fails before any launch
    x = torch.zeros(batch, d_in, dtype=torch.float32, device="cuda")
    y = torch.zeros(batch, d_out, dtype=torch.float32, device="cuda")
    st = N.lib.kq_apply_quantized_noalloc(
        kq.api._ptr(L["packed"]), 2, kq.api._ptr(L["scale"]), kq.api._ptr(L["zero"]), 0,
        kq.api._ptr(x[0]), kq.api._ptr(y[0]), kq.api._ptr(L["sign_in"]), kq.api._ptr(L["sign_out"]),
        0, 0, kq.api._ptr(x), batch, d_out, d_in, kq.api._ptr(y), None)
    assert st == N.KQ_ERR_WORKSPACE
    assert b"scratch" in N.lib.kq_last_error()
