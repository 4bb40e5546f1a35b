"""Streaming capture of a linear layer's KronQ statistics from a torch model.

KronQ summary (hyper.ai), Method: for a linear layer y = W x the weight
gradient of one token is g x^T with g = dL/dy, and under the K-FAC
independence step the empirical Fisher factors as H ~ H_X (x) H_G with
H_X = E[x x^T] and H_G = E[g g^T]; the GPTAQ objective adds the drift between
the layer's input in the full-precision model (X) and in the partly quantized
model (X~). KronQ explainer (gist.science), "Limitazioni": estimating H_G
takes one backward pass over the calibration set.

``CovarianceCapture`` hooks the layer of the full-precision model (its input
on the forward pass, its output gradient on the backward pass) and, when
given, the same layer of the quantized model (its input). Each calibration
batch is one chunk of tokens for ``kq_accumulate_cov`` (beta = 0 for the
first chunk, 1 after, alpha = 1 / n_total): the statistics accumulate on the
device in the library's kernels, and a batch's activations are dropped once
its chunk is in. Nothing here does arithmetic on the statistics.

Conventions:
  * tokens are every leading index of the layer's input (batch, sequence, ...)
    flattened, in the same order for X, X~ and G;
  * bf16 activations go in as bf16 (the kernel's exact products, fp32 sums),
    fp32 as fp32, anything else is converted to fp32;
  * G is the gradient torch delivers for the layer's output, so a loss that
    averages over tokens scales H_G by a constant; that constant is the same
    for every layer of one model and leaves the per-layer solve and the
    bit allocation (which compares sensitivities) unchanged;
  * a layer called more than once per forward pass contributes one token set
    per call (the backward hooks arrive in reverse call order and are paired
    accordingly).

Usage:
    cap = CovarianceCapture(model.layers[3].mlp.down, n_total=N, layer_q=qmodel.layers[3].mlp.down)
    for batch in calibration:
        with cap.batch():
            with torch.no_grad():
                qmodel(batch)                 # X~
            loss_fn(model(batch)).backward()  # X and G
    HX, D, HG = cap.result()
    cap.remove()
"""
from __future__ import annotations

import contextlib

import torch

from . import _native as N
from .api import kq_accumulate_cov, kq_workspace_size


class CovarianceCapture:
    """Accumulates H_X, D and H_G of one linear layer over calibration batches."""

    def __init__(self, layer: torch.nn.Module, n_total: int, layer_q: torch.nn.Module | None = None):
        self.d_in = int(layer.in_features)
        self.d_out = int(layer.out_features)
        if n_total < 1:
            raise ValueError("n_total must be >= 1")
        self.n_total = int(n_total)
        self.seen = 0
        dev = layer.weight.device
        if dev.type != "cuda":
            raise ValueError("the layer must live on the GPU")
        f32 = dict(dtype=torch.float32, device=dev)
        self.HX = torch.zeros(self.d_in, self.d_in, **f32)
        self.D = torch.zeros(self.d_in, self.d_in, **f32) if layer_q is not None else None
        self.HG = torch.zeros(self.d_out, self.d_out, **f32)
        self._x: list[torch.Tensor] = []
        self._xq: list[torch.Tensor] = []
        self._g: list[torch.Tensor] = []
        self._ws = None
        self._has_q = layer_q is not None
        self._hooks = [layer.register_forward_hook(self._on_forward),
                       layer.register_full_backward_hook(self._on_backward)]
        if layer_q is not None:
            if (int(layer_q.in_features), int(layer_q.out_features)) != (self.d_in, self.d_out):
                raise ValueError("layer_q must have the layer's shape")
            self._hooks.append(layer_q.register_forward_hook(self._on_forward_q))

    # hooks: keep detached references only
    def _on_forward(self, mod, inp, out):
        if torch.is_grad_enabled():
            self._x.append(inp[0].detach())

    def _on_forward_q(self, mod, inp, out):
        self._xq.append(inp[0].detach())

    def _on_backward(self, mod, grad_in, grad_out):
        self._g.append(grad_out[0].detach())

    def _tokens(self, t: torch.Tensor, d: int) -> torch.Tensor:
        t = t.reshape(-1, d)
        t = t.contiguous() if t.dtype == torch.bfloat16 else t.to(torch.float32).contiguous()
        if t.data_ptr() % 16:
            t = t.clone()  # the library takes 16-byte aligned buffers
        return t.view(torch.uint16) if t.dtype == torch.bfloat16 else t

    def flush(self) -> int:
        """Send the batch collected so far as one chunk; returns its token count."""
        if not self._x and not self._g and not self._xq:
            return 0
        if len(self._x) != len(self._g):
            raise RuntimeError(f"captured {len(self._x)} forward inputs but {len(self._g)} output "
                               "gradients: run the backward pass inside the batch")
        if self._has_q and len(self._xq) != len(self._x):
            raise RuntimeError(f"captured {len(self._x)} inputs of the layer but {len(self._xq)} of "
                               "the quantized layer")
        xs = self._x
        gs = self._g[::-1]  # backward hooks fire in reverse call order
        xqs = self._xq if self._has_q else xs
        self._x, self._xq, self._g = [], [], []
        X = torch.cat([self._tokens(t, self.d_in) for t in xs]) if len(xs) > 1 else self._tokens(xs[0], self.d_in)
        G = torch.cat([self._tokens(t, self.d_out) for t in gs]) if len(gs) > 1 else self._tokens(gs[0], self.d_out)
        Xq = X if not self._has_q else (
            torch.cat([self._tokens(t, self.d_in) for t in xqs]) if len(xqs) > 1 else self._tokens(xqs[0], self.d_in))
        if not (X.dtype == Xq.dtype == G.dtype):
            # mixed precisions: take all three in fp32
            view = lambda t: t.view(torch.bfloat16).float() if t.dtype == torch.uint16 else t
            X, Xq, G = view(X).contiguous(), view(Xq).contiguous(), view(G).contiguous()
        n = X.shape[0]
        if Xq.shape[0] != n or G.shape[0] != n:
            raise RuntimeError(f"token counts differ: X {n}, X~ {Xq.shape[0]}, G {G.shape[0]}")
        if self.seen + n > self.n_total:
            raise RuntimeError(f"{self.seen + n} tokens captured, more than n_total = {self.n_total}")
        dt = N.KQ_F32 if X.dtype == torch.float32 else N.KQ_BF16
        need = kq_workspace_size(N.KQ_OP_ACCUMULATE_COV, self.d_out, self.d_in, n, dt)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.HX.device)
        kq_accumulate_cov(X if self._has_q else None, Xq, G, 1.0 / self.n_total,
                          0.0 if self.seen == 0 else 1.0, HX=self.HX, D=self.D, HG=self.HG,
                          ws=self._ws)
        self.seen += n
        return n

    @contextlib.contextmanager
    def batch(self):
        """Collect one calibration batch (forward passes and the backward pass)
        and send it as one chunk on exit."""
        if self._x or self._g or self._xq:
            raise RuntimeError("activations from outside a batch() block are pending; flush() first")
        yield self
        self.flush()

    def result(self):
        """(H_X, D, H_G) once n_total tokens are in; D is None without layer_q
        (no drift: X~ = X)."""
        if self.seen != self.n_total:
            raise RuntimeError(f"{self.seen} of {self.n_total} tokens captured")
        return self.HX, self.D, self.HG

    def remove(self):
        for h in self._hooks:
            h.remove()
        self._hooks = []
