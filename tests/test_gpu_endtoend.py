"""End-to-end parity on the LLaMA-2-7B q_proj layer (W 4096 x 4096, 131072
bf16 tokens, 2-bit per-channel grid): the GPU path in the benchmark's launch
configuration against the whole fp64 oracle run on the same inputs.

The oracle accumulates the covariances a token chunk at a time, then runs
BiIP, the sensitivity, the damped inverse factor, P and the column sweep on
its own results; nothing of the GPU's enters it. Compared, with the
tolerances of the comparison protocol:

* covariances, whole matrices: <= 1e-4 relative Frobenius (also per 256 x 256
  tile, so that a wrong low-variance tile cannot hide behind the outliers);
* BiIP outputs, whole and per tile: <= 1e-4;
* sensitivity s = tr(H_G') tr(H_X'): <= 1e-5 relative;
* the layer objective of the GPU's W^ against the oracle's, both evaluated
  by the oracle on its own processed statistics, and the GPU's own objective
  evaluator: <= 1e-3 relative;
* codes: all 16.8M by forced replay on the GPU's own W0', U and P (>= 99.99%
  identical, each mismatch within 1e-4 of a grid step of a midpoint); the
  direct agreement with the oracle's own end-to-end codes is reported.
"""
import time

import numpy as np
import pytest

import oracle
from synth import CHUNK, WORKLOADS, layer_specs, make_layer
from tests.gpu_util import code_report, dev, have_gpu, host, rel_fro, tile_rel_fro

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900),
              pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

if have_gpu():
    import torch

    import post_weight_quantization_amd as kq


def _log(msg):
    print(f"[e2e] {msg}", flush=True)


def test_q_proj_4096_end_to_end_against_the_oracle():
    spec = layer_specs(WORKLOADS["llama2-7b-q_proj"])[0]
    n = spec.n_tok
    t0 = time.time()
    L = make_layer(spec)
    _log(f"inputs {spec.d_out}x{spec.d_in}, N={n} in {time.time() - t0:.1f} s")

    # GPU path, as the benchmark launches it: all tokens in one covariance call
    X, Xq, G = dev(L["x"]), dev(L["xq"]), dev(L["g"])
    HX, D, HG = kq.kq_accumulate_cov(X, Xq, G, 1.0 / n, 0.0)
    del X, Xq, G
    gHX, gD, gHG = host(HX), host(D), host(HG)
    W = dev(L["W"])
    kq.kq_biip(W, HX, D, HG, dev(L["sign_in"]), dev(L["sign_out"]))
    _, _, s_gpu = kq.kq_sensitivity(HX, HG)
    W0p = W.clone()
    U = kq.kq_cholesky_inv(HX, spec.damp)
    P = kq.kq_form_p(D, U)
    codes, scale, zero = kq.kq_gptaq_quantize(W, U, D, spec.bits, spec.group)
    obj_gpu_eval = kq.kq_layer_objective(W0p, W, HX, D, HG)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in dict(HX2=HX, D2=D, HG2=HG, W2=W0p, U=U, P=P, what=W, codes=codes,
                                      scale=scale, zero=zero).items()}
    del HX, D, HG, W, W0p, U, P, codes, scale, zero
    torch.cuda.empty_cache()
    _log("GPU path done")

    # the oracle, end to end on the same token values
    t0 = time.time()
    chunks = ((L["x"][c:c + CHUNK], L["xq"][c:c + CHUNK], L["g"][c:c + CHUNK])
              for c in range(0, n, CHUNK))
    oHX, oD, oHG = oracle.covariances_chunked(chunks, n)
    _log(f"oracle covariances in {time.time() - t0:.1f} s")
    errs = {}
    for name, got, want in (("HX", gHX, oHX), ("D", gD, oD), ("HG", gHG, oHG)):
        errs[name] = rel_fro(got, want)
        errs[name + "_tile"] = tile_rel_fro(got, want, 256)
    _log(f"covariance errors {errs}")
    assert max(errs.values()) <= 1e-4, errs

    t0 = time.time()
    ref = oracle.solve_layer(oHX, oD, oHG, L["W"], L["sign_in"], L["sign_out"], spec.bits,
                             spec.group, spec.block, spec.damp)
    _log(f"oracle BiIP, factor, P and sweep in {time.time() - t0:.1f} s")
    errs = {}
    for name in ("W2", "HX2", "D2", "HG2"):
        errs[name] = rel_fro(g[name], ref[name])
        errs[name + "_tile"] = tile_rel_fro(g[name], ref[name], 256)
    _log(f"BiIP errors {errs}")
    assert max(errs.values()) <= 1e-4, errs

    rel_s = abs(s_gpu / ref["s"] - 1)
    _log(f"s gpu {s_gpu:.9g} oracle {ref['s']:.9g} rel {rel_s:.3g}")
    assert rel_s <= 1e-5

    # objective of the GPU's W^ on the oracle's own processed statistics
    obj_gpu = oracle.objective(ref["W2"], g["what"], ref["HX2"], ref["D2"], ref["HG2"])
    rel_o = abs(obj_gpu / ref["obj"] - 1)
    rel_eval = abs(obj_gpu_eval / ref["obj"] - 1)
    _log(f"objective gpu {obj_gpu:.9g} (own evaluator {obj_gpu_eval:.9g}) oracle {ref['obj']:.9g} "
         f"rel {rel_o:.3g} / {rel_eval:.3g}; round-to-nearest {ref['obj_rtn']:.9g}")
    assert rel_o <= 1e-3 and rel_eval <= 1e-3

    direct = int(np.count_nonzero(g["codes"] != ref["codes"]))
    _log(f"codes differing from the oracle's own end-to-end codes: {direct} of {g['codes'].size} "
         f"({direct / g['codes'].size:.3g}; flips cascade along a row)")

    # every code by forced replay on the GPU's own inputs of the sweep
    t0 = time.time()
    rep_res = oracle.sweep(g["W2"], g["U"].astype(np.float64), g["P"].astype(np.float64), spec.bits,
                           spec.group, spec.block, forced_codes=g["codes"],
                           grid0=(g["scale"][:, 0], g["zero"][:, 0]))
    rep = code_report(rep_res, g["codes"].size)
    _log(f"forced replay of all {g['codes'].size} codes in {time.time() - t0:.1f} s: {rep}")
    assert rep["n"] <= int(1e-4 * g["codes"].size), rep
    assert rep["worst"] <= 1e-4, rep
    sc, zr = oracle.grid_fp32(g["W2"], spec.bits)
    np.testing.assert_array_equal(g["scale"][:, 0], sc)
    np.testing.assert_array_equal(g["zero"][:, 0], zr)
    np.testing.assert_allclose(g["what"], rep_res["what"], rtol=1e-5, atol=1e-6)
