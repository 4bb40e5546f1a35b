"""One layer, and a block of sublayers with mixed precision, chained from the
C-ABI entry points (every step runs in libkq; this module only orders the
calls and holds the buffers).

KronQ summary (hyper.ai), Method: covariances -> BiIP -> sensitivity
s = tr(H_G') tr(H_X') -> column sweep; sublayers with larger s get wider
codes. The sweep never reads H_G (gist.science explainer, Metodologia,
Proposition 1), so it may be freed after the sensitivity.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import api


@dataclass
class Prepared:
    """A sublayer after covariances, BiIP and sensitivity (all on the device)."""

    W: torch.Tensor            # W0' (d_out x d_in fp32), BiIP applied in place
    HX: torch.Tensor           # H_X' (d_in x d_in)
    D: torch.Tensor | None     # D' (d_in x d_in), None without the drift term
    HG: torch.Tensor | None    # H_G' (kept only if asked)
    s_x: torch.Tensor
    s_g: torch.Tensor
    trHX: float
    trHG: float
    s: float
    extra: dict = field(default_factory=dict)

    @property
    def n_params(self) -> int:
        return self.W.shape[0] * self.W.shape[1]


def prepare_layer(X, Xq, G, W, sign_in, sign_out, n_total: int | None = None, keep_hg=False,
                  stream=None) -> Prepared:
    """Covariances over all tokens in one call, BiIP in place on W, sensitivity.

    X may be None (no drift term: plain GPTQ-style objective).
    """
    n = Xq.shape[0] if n_total is None else n_total
    HX, D, HG = api.kq_accumulate_cov(X, Xq, G, 1.0 / n, 0.0, stream=stream,
                                      want=("HX", "D", "HG") if X is not None else ("HX", "HG"))
    s_x, s_g = api.kq_biip(W, HX, D, HG, sign_in, sign_out, stream=stream)
    tx, tg, s = api.kq_sensitivity(HX, HG, stream=stream)
    return Prepared(W=W, HX=HX, D=D, HG=HG if keep_hg else None, s_x=s_x, s_g=s_g, trHX=tx,
                    trHG=tg, s=s)


def quantize_prepared(p: Prepared, bits: int, group: int = 0, damp: float = 0.01,
                      stream=None) -> dict:
    """Inverse factor and sweep; p.W becomes the dequantized W^' in place."""
    U = api.kq_cholesky_inv(p.HX, damp, stream=stream)
    codes, scale, zero = api.kq_gptaq_quantize(p.W, U, p.D, bits, group, stream=stream)
    return dict(U=U, codes=codes, scale=scale, zero=zero)


def allocate(prepared: list[Prepared], widths=(2, 3, 4), avg_budget: float = 2.5) -> list[int]:
    """Widths by descending sensitivity under a parameter-weighted budget."""
    return api.kq_allocate_bits([p.s for p in prepared], [p.n_params for p in prepared], widths,
                                avg_budget)


def quantize_block(prepared: list[Prepared], widths=(2, 3, 4), avg_budget: float = 2.5,
                   group: int = 0, damp: float = 0.01, stream=None):
    """Allocate widths over the block, then quantize every sublayer with its width."""
    bits = allocate(prepared, widths, avg_budget)
    out = [quantize_prepared(p, b, group, damp, stream) for p, b in zip(prepared, bits)]
    return bits, out


__all__ = ["Prepared", "prepare_layer", "quantize_prepared", "allocate", "quantize_block"]
