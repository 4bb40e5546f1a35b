"""Seeded synthetic calibration data for one linear layer y = W x.

The pages measure KronQ on LLaMA-family checkpoints with WikiText-2 / C4 style
calibration sets; neither is available here, so every input is drawn from the
distributions below, which stand in for them (shapes of the LLaMA-2-7B,
LLaMA-3-70B projections, heavy-tailed per-channel activation scales with a few
outlier channels, output-gradient scales spread over orders of magnitude as the
KronQ summary (hyper.ai), Method, figure on normalised diag(H_G), describes):

* sigma_j ~ LogNormal(0, 1) per input channel; the first ``n_outlier`` channels
  are multiplied by 20.
* X rows ~ N(0, diag(sigma^2)); the quantized model's input is
  X~ = X + N(0, (0.01 sigma)^2), drawn from an independent stream.
* tau_i ~ LogNormal(0, 2) per output channel; G rows ~ N(0, diag(tau^2)).
* W ~ N(0, 0.02^2) as fp32 master weights.
* Random signs for the two randomized Hadamard transforms, +-1 as int8.

Tokens are drawn in chunks of ``CHUNK`` rows, each from its own seeded PCG64
stream keyed by ``SeedSequence([workload, stream, index, chunk])``, so any
prefix, any chunk and any subset of chunks can be regenerated independently
and in parallel. For the bf16 workloads the fp32 draw is rounded to bf16 with
round-to-nearest-even and stored as its 16-bit pattern (uint16); both the
oracle and the GPU path then read the identical values.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

CHUNK = 8192

# stream identifiers inside a workload's seed sequence
_S_SIGMA, _S_TAU, _S_W, _S_X, _S_NOISE, _S_G, _S_SIGN_IN, _S_SIGN_OUT = range(1, 9)


@dataclass(frozen=True)
class LayerSpec:
    """One linear layer of a workload (all sizes in elements)."""

    cfg: int          # workload index
    name: str         # sublayer name
    d_out: int
    d_in: int
    n_tok: int
    dtype: str        # "f32" or "bf16" for X, X~ and G
    bits: int         # code width
    group: int        # 0: one grid per output channel; else columns per group
    block: int        # lazy-update block of the column sweep
    damp: float       # damping as a fraction of mean(diag H_X)
    n_outlier: int    # number of outlier input channels (x20)
    x_stream: int     # activation stream index (shared by sublayers reading the same X)
    g_stream: int     # gradient stream index (one per sublayer)
    sub: int          # sublayer index inside the workload (keys W and the signs)

    @property
    def n_params(self) -> int:
        return self.d_out * self.d_in

    def with_tokens(self, n_tok: int) -> "LayerSpec":
        return replace(self, n_tok=n_tok)


def _spec(cfg, name, d_out, d_in, *, n_tok=131072, dtype="bf16", bits=2, group=0,
          n_outlier=16, x_stream=0, g_stream=0, sub=0):
    return LayerSpec(cfg=cfg, name=name, d_out=d_out, d_in=d_in, n_tok=n_tok, dtype=dtype,
                     bits=bits, group=group, block=128, damp=0.01, n_outlier=n_outlier,
                     x_stream=x_stream, g_stream=g_stream, sub=sub)


# Workloads. 0: tiny fp32 layer; 1: LLaMA-2-7B q_proj; 2: LLaMA-2-7B MLP (3-bit,
# groups of 128); 3: LLaMA-3-70B q_proj and down_proj; 4: a full LLaMA-3-70B
# decoder block whose widths come from the mixed-precision allocation.
CONFIGS: dict[int, list[LayerSpec]] = {
    0: [_spec(0, "toy", 256, 256, n_tok=1024, dtype="f32", n_outlier=4)],
    1: [_spec(1, "q_proj", 4096, 4096)],
    2: [_spec(2, "gate_proj", 11008, 4096, bits=3, group=128, x_stream=0, g_stream=0, sub=0),
        _spec(2, "up_proj", 11008, 4096, bits=3, group=128, x_stream=0, g_stream=1, sub=1),
        _spec(2, "down_proj", 4096, 11008, bits=3, group=128, x_stream=1, g_stream=2, sub=2)],
    3: [_spec(3, "q_proj", 8192, 8192, x_stream=0, g_stream=0, sub=0),
        _spec(3, "down_proj", 8192, 28672, x_stream=1, g_stream=1, sub=1)],
    4: [_spec(4, "q_proj", 8192, 8192, x_stream=0, g_stream=0, sub=0),
        _spec(4, "k_proj", 1024, 8192, x_stream=0, g_stream=1, sub=1),
        _spec(4, "v_proj", 1024, 8192, x_stream=0, g_stream=2, sub=2),
        _spec(4, "o_proj", 8192, 8192, x_stream=1, g_stream=3, sub=3),
        _spec(4, "gate_proj", 28672, 8192, x_stream=2, g_stream=4, sub=4),
        _spec(4, "up_proj", 28672, 8192, x_stream=2, g_stream=5, sub=5),
        _spec(4, "down_proj", 8192, 28672, x_stream=3, g_stream=6, sub=6)],
}

# names of the workloads, as used on command lines
WORKLOADS: dict[str, int] = {
    "toy-256": 0,
    "llama2-7b-q_proj": 1,
    "llama2-7b-mlp": 2,
    "llama3-70b-q-down": 3,
    "llama3-70b-block": 4,
}

# average bits per parameter available to the decoder block of workload 4
BLOCK_BUDGET_BITS = 2.5
BLOCK_WIDTHS = (2, 3, 4)


def layer_specs(cfg: int) -> list[LayerSpec]:
    return list(CONFIGS[cfg])


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, nearest-even, returning the 16-bit patterns (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _sigma(spec: LayerSpec) -> np.ndarray:
    s = _rng(spec.cfg, _S_SIGMA, spec.x_stream).lognormal(0.0, 1.0, spec.d_in).astype(np.float32)
    s[: spec.n_outlier] *= np.float32(20.0)
    return s


def _tau(spec: LayerSpec) -> np.ndarray:
    return _rng(spec.cfg, _S_TAU, spec.g_stream).lognormal(0.0, 2.0, spec.d_out).astype(np.float32)


def token_chunk(spec: LayerSpec, which: str, c: int, rows: int | None = None) -> np.ndarray:
    """Rows [c*CHUNK, c*CHUNK + rows) of X ("x"), X~ ("xq") or G ("g").

    Returns float32 for fp32 workloads and uint16 bf16 patterns otherwise.
    """
    n = min(CHUNK, spec.n_tok - c * CHUNK) if rows is None else rows
    if which == "g":
        z = _rng(spec.cfg, _S_G, spec.g_stream, c).standard_normal((n, spec.d_out), dtype=np.float32)
        out = z * _tau(spec)[None, :]
    else:
        sig = _sigma(spec)
        x = _rng(spec.cfg, _S_X, spec.x_stream, c).standard_normal((n, spec.d_in), dtype=np.float32)
        x *= sig[None, :]
        if which == "x":
            out = x
        elif which == "xq":
            nz = _rng(spec.cfg, _S_NOISE, spec.x_stream, c).standard_normal((n, spec.d_in), dtype=np.float32)
            nz *= (np.float32(0.01) * sig)[None, :]
            out = x + nz
        else:
            raise ValueError(which)
    if spec.dtype == "f32":
        return np.ascontiguousarray(out, dtype=np.float32)
    return f32_to_bf16_bits(out)


def _stack(spec: LayerSpec, which: str, n_tok: int, threads: int) -> np.ndarray:
    width = spec.d_out if which == "g" else spec.d_in
    dt = np.float32 if spec.dtype == "f32" else np.uint16
    out = np.empty((n_tok, width), dtype=dt)
    n_chunks = (n_tok + CHUNK - 1) // CHUNK

    def fill(c):
        r0 = c * CHUNK
        rows = min(CHUNK, n_tok - r0)
        out[r0:r0 + rows] = token_chunk(spec, which, c, rows)

    if n_chunks == 1 or threads <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def make_weights(spec: LayerSpec) -> np.ndarray:
    w = _rng(spec.cfg, _S_W, spec.sub).standard_normal((spec.d_out, spec.d_in), dtype=np.float32)
    return w * np.float32(0.02)


def make_signs(spec: LayerSpec) -> tuple[np.ndarray, np.ndarray]:
    """(sign_in over d_in, sign_out over d_out), each +-1 int8."""
    si = _rng(spec.cfg, _S_SIGN_IN, spec.sub).integers(0, 2, spec.d_in).astype(np.int8) * 2 - 1
    so = _rng(spec.cfg, _S_SIGN_OUT, spec.sub).integers(0, 2, spec.d_out).astype(np.int8) * 2 - 1
    return si.astype(np.int8), so.astype(np.int8)


def make_layer(spec: LayerSpec, n_tok: int | None = None, threads: int | None = None,
               parts=("x", "xq", "g")) -> dict:
    """All inputs of one layer: X, Xq (X~), G token-major, W, sign vectors.

    ``n_tok`` takes a prefix of the token stream (the chunks are the same).
    """
    n = spec.n_tok if n_tok is None else n_tok
    th = threads if threads is not None else min(16, os.cpu_count() or 1)
    out = {"spec": spec, "n_tok": n, "W": make_weights(spec)}
    out["sign_in"], out["sign_out"] = make_signs(spec)
    for p in parts:
        out[p] = _stack(spec, p, n, th)
    return out
