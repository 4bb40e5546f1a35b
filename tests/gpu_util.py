"""Helpers shared by the GPU parity tests (comparison metrics, device moves)."""
from __future__ import annotations

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def have_gpu() -> bool:
    return torch is not None and torch.cuda.is_available()


def dev(a, dtype=None):
    """numpy -> contiguous cuda tensor (uint16 stays uint16: bf16 bit patterns)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.uint16)
    else:
        t = torch.from_numpy(a if dtype is None else a.astype(dtype))
    return t.cuda()


def host(t) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.uint16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def spd(rng, n, cond=100.0):
    q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    ev = np.exp(rng.uniform(0, np.log(cond), n))
    return (q * ev) @ q.T


def code_report(res, n_total):
    """Summary of a forced replay: mismatch count, worst midpoint distance."""
    mm = res["mismatches"]
    worst = max((m[4] for m in mm), default=0.0)
    return dict(n=len(mm), frac=len(mm) / n_total, worst=worst)


def tile_rel_fro(a, b, t: int) -> float:
    """Largest relative Frobenius error over the t x t tiles of a matrix
    (rows of t entries for vectors): a wrong tile of small values fails
    even when larger tiles dominate the whole matrix's norm. Tiles whose
    reference is zero must match it exactly."""
    a = np.atleast_2d(np.asarray(a, np.float64))
    b = np.atleast_2d(np.asarray(b, np.float64))
    worst = 0.0
    for i in range(0, b.shape[0], t):
        for j in range(0, b.shape[1], t):
            rb = np.linalg.norm(b[i:i + t, j:j + t])
            ra = np.linalg.norm(a[i:i + t, j:j + t] - b[i:i + t, j:j + t])
            worst = max(worst, ra / rb if rb > 0 else (0.0 if ra == 0 else np.inf))
    return float(worst)
