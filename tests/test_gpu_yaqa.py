"""GPU parity of the rounding with output-side feedback (kq_yaqa_quantize)
against oracle/yaqa.py.

Codes are integers decided in floating point: the GPU rounds fp32 fed-back
inputs and the oracle fp64 ones, so codes are compared by forced replay
(the bar of the KronQ sweep): at most 1e-4 of the codes may differ, and each
that differs must have an oracle input within 1e-4 grid steps of the
midpoint between the two codes. Grids are bit-exact (fp32 on both sides from
the same W0). Inputs for both sides come from the oracle (fp64 factors
rounded to fp32).

At full size the oracle's row-major rounding would take hours, so the GPU
result is checked by a property that holds at any size: the rounding
residuals solved back from (W*, W^) (oracle.yaqa.residuals_of) lie within
half a grid step, to 1e-4 of a step — every code is the rounding of its own
fed-back input.
"""
import numpy as np
import pytest

import oracle
from oracle import yaqa
from tests.gpu_util import code_report, dev, have_gpu, host, rel_fro, spd

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

if have_gpu():
    import post_weight_quantization_amd as kq


def _run_gpu(W0, UI, UO, D, bits):
    tW = dev(W0)
    codes, scale, zero = kq.kq_yaqa_quantize(tW, dev(UI), dev(UO), dev(D) if D is not None else None,
                                             bits)
    return host(codes), host(scale)[:, 0], host(zero)[:, 0], host(tW)


def _check_replay(W0, UI, UO, D, bits, codes, scale, zero, What):
    P = oracle.form_p(D, UI) if D is not None else None
    ref = yaqa.quantize_two_sided(W0, UI, UO, bits, P=P, forced_codes=codes)
    rep = code_report(ref, codes.size)
    assert rep["n"] <= max(1, int(1e-4 * codes.size)), rep
    assert rep["worst"] <= 1e-4, rep
    sc, zr = oracle.grid_fp32(W0, bits)
    np.testing.assert_array_equal(scale, sc)
    np.testing.assert_array_equal(zero, zr)
    np.testing.assert_allclose(What, scale[:, None] * (codes.astype(np.float32) - zero[:, None]),
                               rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(What, ref["what"], rtol=1e-5, atol=1e-6)
    return ref


def _case(d_out, d_in, with_d, seed):
    rng = np.random.default_rng(seed)
    UI = oracle.inv_factor(spd(rng, d_in, 1e3), 0.01).astype(np.float32)
    UO = oracle.inv_factor(spd(rng, d_out, 1e3), 0.01).astype(np.float32)
    D = (0.02 * rng.standard_normal((d_in, d_in))).astype(np.float32) if with_d else None
    W0 = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    return W0, UI, UO, D


# one tile; several tiles; ragged both ways; one row; one column; one entry
@pytest.mark.parametrize("d_out,d_in,bits,with_d", [
    (64, 64, 2, False), (128, 192, 2, True), (256, 256, 3, True), (200, 300, 3, False),
    (130, 70, 4, True), (1, 200, 2, False), (150, 1, 3, False), (1, 1, 2, False),
    (65, 129, 8, True)])
def test_yaqa_forced_replay(d_out, d_in, bits, with_d):
    W0, UI, UO, D = _case(d_out, d_in, with_d, 7 * d_out + d_in)
    codes, scale, zero, What = _run_gpu(W0, UI, UO, D, bits)
    _check_replay(W0, UI, UO, D, bits, codes, scale, zero, What)


def test_yaqa_zero_rows_and_repeat_calls():
    """All-zero rows take the [-1, 1] grid; a second call on the same
    buffers after a larger one gives the same result as a fresh one."""
    W0, UI, UO, D = _case(96, 160, True, 3)
    W0[5] = 0.0
    W0[64:70] = 0.0
    big = _case(300, 320, True, 4)
    _run_gpu(*big, 2)
    first = _run_gpu(W0, UI, UO, D, 2)
    second = _run_gpu(W0, UI, UO, D, 2)
    for a, b in zip(first, second):
        np.testing.assert_array_equal(a, b)
    _check_replay(W0, UI, UO, D, 2, *first)


def test_yaqa_identity_output_is_the_sweep():
    """With U_out = I the rounding is the KronQ sweep: the GPU result is
    replayed against the oracle's GPTAQ sweep as well."""
    W0, UI, _, D = _case(96, 256, True, 9)
    codes, scale, zero, What = _run_gpu(W0, UI, np.eye(96, dtype=np.float32), D, 2)
    ref = oracle.sweep(W0, UI, oracle.form_p(D, UI), 2, 0, 128, forced_codes=codes)
    rep = code_report(ref, codes.size)
    assert rep["n"] <= max(1, int(1e-4 * codes.size)) and rep["worst"] <= 1e-4, rep
    np.testing.assert_allclose(What, ref["what"], rtol=1e-5, atol=1e-6)


def test_yaqa_on_the_toy_layer():
    """The toy workload through the oracle's covariances and BiIP, then the
    GPU rounding with U_in from H_X' and U_out from H_G'; on this layer the
    output feedback lowers the layer objective well below the one-sided
    sweep's."""
    from synth import layer_specs, make_layer
    spec = layer_specs(0)[0]
    L = make_layer(spec)
    HX, D, HG = oracle.covariances(L["x"], L["xq"], L["g"])
    W2, HX2, D2, HG2 = oracle.biip(L["W"], HX, D, HG, L["sign_in"], L["sign_out"])[:4]
    UI = oracle.inv_factor(HX2, spec.damp).astype(np.float32)
    UO = oracle.inv_factor(HG2, spec.damp).astype(np.float32)
    W0 = W2.astype(np.float32)
    D32 = D2.astype(np.float32)
    codes, scale, zero, What = _run_gpu(W0, UI, UO, D32, spec.bits)
    _check_replay(W0, UI, UO, D32, spec.bits, codes, scale, zero, What)
    one = oracle.sweep(W0, UI, oracle.form_p(D32, UI), spec.bits, 0, 128)
    obj_two = oracle.objective(W0, What, HX2, D2, HG2)
    obj_one = oracle.objective(W0, one["what"], HX2, D2, HG2)
    print(f"layer objective: two-sided {obj_two:.4g}, one-sided {obj_one:.4g}")
    assert obj_two < 0.5 * obj_one


@pytest.mark.slow
@pytest.mark.parametrize("d_out,d_in,with_d", [(4096, 4096, True), (1000, 4100, False),
                                                (8192, 8192, True)])
def test_yaqa_full_size_residuals(d_out, d_in, with_d):
    """The bench layer's shape (2-bit, one grid per channel), a ragged one and
    the 70B q_proj shape: every residual solved back from the result lies
    within half a grid step (1e-4 of a step of slack for fp32)."""
    rng = np.random.default_rng(d_out + d_in)
    print(f"[yaqa full] {d_out}x{d_in} D={with_d}: factors", flush=True)
    UI = oracle.inv_factor(spd(rng, d_in, 1e3), 0.01).astype(np.float32)
    UO = oracle.inv_factor(spd(rng, d_out, 1e3), 0.01).astype(np.float32)
    D = (0.02 * rng.standard_normal((d_in, d_in))).astype(np.float32) if with_d else None
    W0 = (0.02 * rng.standard_normal((d_out, d_in))).astype(np.float32)
    print("[yaqa full] GPU rounding", flush=True)
    codes, scale, zero, What = _run_gpu(W0, UI, UO, D, 2)
    print("[yaqa full] residuals", flush=True)
    Wt = W0.astype(np.float64)
    if with_d:
        Wt = Wt + Wt @ oracle.form_p(D, UI)
    eps = yaqa.residuals_of(Wt, What, UI, UO)
    viol = yaqa.rounding_violation(eps, codes, scale, 2)
    print(f"[yaqa full] worst excess over half a step: {viol:.3g} steps", flush=True)
    assert viol <= 1e-4
    np.testing.assert_array_equal(scale, oracle.grid_fp32(W0, 2)[0])
