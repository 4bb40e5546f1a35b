"""GPU parity of the streaming statistics capture (capture.py) against the
oracle's covariances of the concatenated token stream.

A small random-initialised two-layer MLP stands in for a model (no trained
weights: the capture is plumbing around kq_accumulate_cov, and only the
statistics are compared). The quantized model is a copy whose first layer's
weights are rounded to a coarse grid, so the second layer's input drifts.
Independent plain hooks in the test keep host copies of X, X~ and G; the
oracle (oracle.covariances, fp64) computes H_X, D and H_G from their
concatenation, and the capture, fed batch by batch, must agree to the
covariance tolerance of the other parity tests (1e-4 relative Frobenius).
"""
import copy

import numpy as np
import pytest

import oracle
from tests.gpu_util import have_gpu, rel_fro

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

if have_gpu():
    import torch

    import post_weight_quantization_amd as kq


def _models(dtype, d_in=256, d_hid=512, d_out=256, seed=0):
    torch.manual_seed(seed)
    model = torch.nn.Sequential(torch.nn.Linear(d_in, d_hid), torch.nn.GELU(),
                                torch.nn.Linear(d_hid, d_out)).to("cuda", dtype)
    qmodel = copy.deepcopy(model)
    with torch.no_grad():
        w = qmodel[0].weight
        step = (w.float().abs().max() / 3).item()
        w.copy_((torch.round(w.float() / step) * step).to(dtype))
    return model, qmodel


def _host(t):
    t = t.detach().reshape(-1, t.shape[-1])
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.uint16).cpu().numpy()
    return t.float().cpu().numpy()


@pytest.mark.parametrize("dtype,batches,shape", [("bf16", 3, (4, 96)), ("f32", 2, (2, 64)),
                                                  ("bf16", 1, (1, 24))])
def test_capture_matches_oracle(dtype, batches, shape):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    model, qmodel = _models(dt)
    layer, layer_q = model[2], qmodel[2]
    n_total = batches * shape[0] * shape[1]
    cap = kq.CovarianceCapture(layer, n_total, layer_q=layer_q)
    seen = {"x": [], "xq": [], "g": []}
    hs = [layer.register_forward_hook(lambda m, i, o: seen["x"].append(_host(i[0]))),
          layer_q.register_forward_hook(lambda m, i, o: seen["xq"].append(_host(i[0]))),
          layer.register_full_backward_hook(lambda m, gi, go: seen["g"].append(_host(go[0])))]
    gen = torch.Generator(device="cuda").manual_seed(1)
    for _ in range(batches):
        inp = torch.randn(*shape, 256, device="cuda", generator=gen).to(dt)
        labels = torch.randint(0, 256, shape, device="cuda", generator=gen)
        with cap.batch():
            with torch.no_grad():
                qmodel(inp)
            logits = model(inp)
            loss = torch.nn.functional.cross_entropy(logits.float().reshape(-1, 256), labels.reshape(-1))
            loss.backward()
    HX, D, HG = cap.result()
    cap.remove()
    for h in hs:
        h.remove()
    X, Xq, G = (np.concatenate(seen[k]) for k in ("x", "xq", "g"))
    assert X.shape == (n_total, 512) and G.shape == (n_total, 256)
    wHX, wD, wHG = oracle.covariances(X, Xq, G)
    torch.cuda.synchronize()
    assert rel_fro(HX.cpu().numpy(), wHX) < 1e-4
    assert rel_fro(D.cpu().numpy(), wD) < 1e-4
    assert rel_fro(HG.cpu().numpy(), wHG) < 1e-4
    assert np.abs(wD).max() > 0  # the quantized copy really drifts


def test_capture_without_quantized_model_and_counts():
    model, _ = _models(torch.bfloat16, seed=3)
    layer = model[2]
    cap = kq.CovarianceCapture(layer, 2 * 48)
    X, G = [], []
    hs = [layer.register_forward_hook(lambda m, i, o: X.append(_host(i[0]))),
          layer.register_full_backward_hook(lambda m, gi, go: G.append(_host(go[0])))]
    gen = torch.Generator(device="cuda").manual_seed(4)
    for k in range(2):
        inp = torch.randn(48, 256, device="cuda", generator=gen).to(torch.bfloat16)
        with cap.batch():
            model(inp).float().square().mean().backward()
        if k == 0:
            with pytest.raises(RuntimeError, match="48 of 96"):
                cap.result()
    HX, D, HG = cap.result()
    assert D is None
    wHX, _, wHG = oracle.covariances(None, np.concatenate(X), np.concatenate(G))
    assert rel_fro(HX.cpu().numpy(), wHX) < 1e-4
    assert rel_fro(HG.cpu().numpy(), wHG) < 1e-4
    # one more batch would exceed n_total
    inp = torch.randn(8, 256, device="cuda", generator=gen).to(torch.bfloat16)
    with pytest.raises(RuntimeError, match="more than n_total"):
        with cap.batch():
            model(inp).float().square().mean().backward()
    # a forward without its backward inside a batch is an error
    cap2 = kq.CovarianceCapture(layer, 8)
    with pytest.raises(RuntimeError, match="output gradients"):
        with cap2.batch():
            model(inp)
    cap.remove()
    cap2.remove()
    for h in hs:
        h.remove()
