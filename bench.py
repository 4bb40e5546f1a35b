"""Benchmark: KronQ layer quantization on one MI355X.

One step is the whole per-layer hot path on device-resident inputs:
covariances (H_X, D, H_G) -> BiIP -> sensitivity -> inverse factor -> GPTAQ
sweep, for the LLaMA-2-7B q_proj workload (W 4096 x 4096, 131072 bf16
calibration tokens, 2-bit per-channel grid, lazy block 128, 1% damping, full
4096-point randomized Hadamard on both sides). The metric is milliseconds per
layer (lower is better). Per-stage times come from HIP events recorded on the
stream the kernels run on; the covariance kernel, the dominant one, is also
timed alone through the library's event hook. The CPU baseline is the fp64
oracle timed on a bounded sample of the same workload on this host's cores.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2] [--workload llama2-7b-q_proj]
                    [--no-cpu] [--copy-calib MIB]

--copy-calib runs one device-to-device copy of MIB mebibytes before the steps,
so that a hardware-counter pass over the same command sees a kernel of known
traffic next to the covariance kernel (the scaling factor for FETCH_SIZE and
WRITE_SIZE).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15      # dense MFMA, FLOP/s
PEAK_FP32_MFMA = 157.3e12
PEAK_HBM = 8.0e12       # bytes/s

# HBM traffic of one covariance-kernel launch on the LLaMA-2-7B q_proj
# workload (4096 x 4096, 131072 bf16 tokens), from FETCH_SIZE and WRITE_SIZE
# counter passes scaled by the same counters on a copy of known size. Valid
# only for the kernel source it was measured on (sha256 of cov.hip).
COV_TRAFFIC = {"cov_sha256": "fe94307568c79ebd377fe637262b97325f7c45a8555dbc8bc7172fbbb4343543",
               "bytes": 17111960064}


def stage_costs(spec):
    """Algorithmic flops / bytes of each stage (triangles exploited; 2 flops per FMA)."""
    n, m, N = spec.d_in, spec.d_out, spec.n_tok
    cov_flops = n * (n + 1) * N + 2 * n * n * N + m * (m + 1) * N
    # BiIP: two single-side passes (read + write fp32) over W, H_X, D, H_G, plus one read of W for norms
    biip_bytes = 16 * (m * n + 2 * n * n + m * m) + 4 * m * n
    # its floor: every element of W, H_X, D, H_G read once and written once
    biip_min_bytes = 8 * (m * n + 2 * n * n + m * m)
    chol_flops = 2 * n ** 3 / 3                     # Cholesky n^3/3 + triangular inverse n^3/3
    solve_flops = 2 * n ** 3 / 3 + 2 * m * n * n    # P formation + fold W0 P (P strictly upper) + trailing updates
    return dict(cov_flops=cov_flops, biip_bytes=biip_bytes, biip_min_bytes=biip_min_bytes,
                chol_flops=chol_flops, solve_flops=solve_flops)


def run_gpu(spec, steps, warmup, data, extras=True):
    import torch

    import post_weight_quantization_amd as kq
    from post_weight_quantization_amd import _native as N

    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).to(dev)
    X, Xq, G = t(data["x"]), t(data["xq"]), t(data["g"])
    if data["x"].dtype == np.uint16:
        X, Xq, G = X.view(torch.uint16), Xq.view(torch.uint16), G.view(torch.uint16)
    W0 = t(data["W"])
    si, so = t(data["sign_in"]), t(data["sign_out"])
    n, m = spec.d_in, spec.d_out
    f32 = dict(dtype=torch.float32, device=dev)
    HX, D, HG = torch.empty(n, n, **f32), torch.empty(n, n, **f32), torch.empty(m, m, **f32)
    U = torch.empty(n, n, **f32)
    W = torch.empty_like(W0)
    s_x, s_g = torch.empty(n, **f32), torch.empty(m, **f32)
    ng = n // spec.group if spec.group else 1
    codes = torch.empty(m, n, dtype=torch.uint8, device=dev)
    scale, zero = torch.empty(m, ng, **f32), torch.empty(m, ng, **f32)
    dt = N.KQ_F32 if spec.dtype == "f32" else N.KQ_BF16
    cfg = N.kq_quant_cfg(spec.bits, spec.group, spec.block, 0)
    need = max(kq.kq_workspace_size(N.KQ_OP_ACCUMULATE_COV, m, n, spec.n_tok, dt),
               kq.kq_workspace_size(N.KQ_OP_BIIP, m, n),
               kq.kq_workspace_size(N.KQ_OP_SENSITIVITY, m, n),
               kq.kq_workspace_size(N.KQ_OP_CHOLESKY_INV, n, n),
               kq.kq_workspace_size(N.KQ_OP_GPTAQ_QUANTIZE, m, n, cfg=cfg))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    names = ["cov", "biip", "chol", "gptaq", "sens"]
    stream = torch.cuda.current_stream()
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(ev=None, k=None):
        W.copy_(W0)
        if k is not None:
            kq.kq_set_kernel_events(N.KQ_OP_ACCUMULATE_COV, kev[k][0], kev[k][1], stream)
        if ev: ev[0].record(stream)
        kq.kq_accumulate_cov(X, Xq, G, 1.0 / spec.n_tok, 0.0, HX, D, HG, ws=ws)
        if k is not None:
            kq.kq_set_kernel_events(N.KQ_OP_ACCUMULATE_COV)
        if ev: ev[1].record(stream)
        kq.kq_biip(W, HX, D, HG, si, so, 0, 0, s_x, s_g, ws=ws)
        if ev: ev[2].record(stream)
        kq.kq_cholesky_inv(HX, spec.damp, U, ws=ws)
        if ev: ev[3].record(stream)
        if k is not None:
            kq.kq_set_kernel_events(N.KQ_OP_GPTAQ_QUANTIZE, kev[k][2], kev[k][3], stream)
        kq.kq_gptaq_quantize(W, U, D, spec.bits, spec.group, spec.block, codes, scale, zero, ws=ws)
        if k is not None:
            kq.kq_set_kernel_events(N.KQ_OP_GPTAQ_QUANTIZE)
        if ev: ev[4].record(stream)
        # the sensitivity reads only HX and HG (final after BiIP) and returns
        # host values; called last so that its wait falls at the end of the
        # step instead of between two stages
        out = kq.kq_sensitivity(HX, HG, ws=ws)
        if ev: ev[5].record(stream)
        return out

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    # create the hook's events before the timed region
    for k in range(steps):
        for e in kev[k]:
            e.record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        sens = step(evs[k], k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {nm: float(np.mean([evs[k][i].elapsed_time(evs[k][i + 1]) for k in range(steps)]))
                for i, nm in enumerate(names)}
    cov_kernel_ms = float(np.mean([kev[k][0].elapsed_time(kev[k][1]) for k in range(steps)]))
    trail_kernel_ms = (float(np.mean([kev[k][2].elapsed_time(kev[k][3]) for k in range(steps)]))
                       if spec.d_in > 512 else None)
    # quality check outside the timed region
    W0p = None
    obj = None
    try:
        # re-run the front half once to get W0' for the objective
        W.copy_(W0)
        kq.kq_accumulate_cov(X, Xq, G, 1.0 / spec.n_tok, 0.0, HX, D, HG, ws=ws)
        kq.kq_biip(W, HX, D, HG, si, so, 0, 0, s_x, s_g, ws=ws)
        W0p = W.clone()
        kq.kq_cholesky_inv(HX, spec.damp, U, ws=ws)
        kq.kq_gptaq_quantize(W, U, D, spec.bits, spec.group, spec.block, codes, scale, zero, ws=ws)
        obj = kq.kq_layer_objective(W0p, W, HX, D, HG)
        Wr = W0p.clone()
        # round-to-nearest on the same grid, for reference
        if not spec.group:
            Wr = scale * (torch.clamp(torch.round(W0p / scale) + zero, 0, 2 ** spec.bits - 1) - zero)
            obj_rtn = kq.kq_layer_objective(W0p, Wr.contiguous(), HX, D, HG)
        else:
            obj_rtn = None
    except Exception as e:  # pragma: no cover - reporting only
        print(f"objective check failed: {e}", file=sys.stderr)
        obj_rtn = None
    inf = fb = cap = None
    if extras:
        inf = run_inference(spec, codes, scale, zero, s_x, s_g, si, so)
        fb = run_output_feedback(spec, W0p, HX, D, HG, U, obj) if W0p is not None and not spec.group else None
        cap = run_streaming(spec, X, Xq, G, HX, D, HG, ws)
    return dict(wall_s=wall, stage_ms=stage_ms, cov_kernel_ms=cov_kernel_ms, trail_kernel_ms=trail_kernel_ms,
                sens=sens, obj=obj,
                obj_rtn=obj_rtn, inference=inf, streaming=cap, output_feedback=fb)


def run_output_feedback(spec, W0p, HX, D, HG, U, obj_gptaq, reps=3):
    """The rounding with output-side feedback (generalized LDLQ on H_G' x H_X')
    on the same processed layer: U_out from H_G', the GPTAQ fold as target.
    Time per call (to the end of its last kernel), its algorithmic flops, and the
    layer objective beside the one-sided sweep's."""
    import torch

    import post_weight_quantization_amd as kq
    from post_weight_quantization_amd import _native as N

    m, n = spec.d_out, spec.d_in
    stream = torch.cuda.current_stream()
    cfg = N.kq_quant_cfg(spec.bits, 0, 128, 0)
    ws = torch.empty(max(kq.kq_workspace_size(N.KQ_OP_YAQA_QUANTIZE, m, n, cfg=cfg),
                         kq.kq_workspace_size(N.KQ_OP_CHOLESKY_INV, m, m)), dtype=torch.uint8,
                     device=W0p.device)
    Uo = torch.empty(m, m, dtype=torch.float32, device=W0p.device)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    kq.kq_cholesky_inv(HG, spec.damp, Uo, ws=ws)
    ev[1].record(stream)
    torch.cuda.synchronize()
    chol_ms = ev[0].elapsed_time(ev[1])
    W = W0p.clone()
    kq.kq_yaqa_quantize(W, U, Uo, D, spec.bits, ws=ws)  # warm-up
    ts = []
    for _ in range(reps):
        W.copy_(W0p)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        kq.kq_yaqa_quantize(W, U, Uo, D, spec.bits, ws=ws)
        torch.cuda.synchronize()
        ts.append(time.perf_counter() - t0)
    ms = 1e3 * float(np.median(ts))
    obj = kq.kq_layer_objective(W0p, W, HX, D, HG)
    # row feedback m n^2, column feedback m^2 n, P formation 2 n^3 / 3, fold m n^2 (2 flops per FMA)
    flops = m * n * n + m * m * n + 2 * n ** 3 / 3 + m * n * n
    return {"ms": round(ms, 3), "tflops": round(flops / ms / 1e9, 2),
            "frac_fp32_mfma": round(flops / (ms * 1e-3) / PEAK_FP32_MFMA, 3),
            "u_out_factor_ms": round(chol_ms, 3),
            "objective": obj, "objective_one_sided": obj_gptaq}


def run_streaming(spec, X, Xq, G, HX, D, HG, ws, chunk=16384, reps=3):
    """Covariances of the same tokens streamed in chunks (the way a capture
    of calibration batches feeds them: beta = 0, then 1) against one call."""
    import torch

    import post_weight_quantization_amd as kq

    from post_weight_quantization_amd import _native as N

    n = spec.n_tok
    if n % chunk:
        return None
    stream = torch.cuda.current_stream()
    dt = N.KQ_F32 if spec.dtype == "f32" else N.KQ_BF16
    need = max(kq.kq_workspace_size(N.KQ_OP_ACCUMULATE_COV, spec.d_out, spec.d_in, c, dt) for c in (n, chunk))
    if ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=ws.device)

    def once(c):
        for k in range(0, n, c):
            kq.kq_accumulate_cov(X[k:k + c], Xq[k:k + c], G[k:k + c], 1.0 / n, 0.0 if k == 0 else 1.0,
                                 HX, D, HG, ws=ws)

    res = {}
    for c in (n, chunk):
        once(c)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(reps):
            once(c)
        ev[1].record(stream)
        torch.cuda.synchronize()
        res[c] = ev[0].elapsed_time(ev[1]) / reps
    return {"tokens": n, "chunk_tokens": chunk, "chunks": n // chunk,
            "chunked_ms": round(res[chunk], 3), "single_call_ms": round(res[n], 3),
            "chunked_mtok_s": round(n / res[chunk] / 1e3, 2)}


_SPIN = {}


def hold_gpu(ms=0.5):
    """Enqueue a spin kernel of about `ms` milliseconds on the current stream,
    so that the host queues the call that follows before the GPU reaches it:
    its events then time the GPU's work, not the host's launches."""
    import torch

    if "per_ms" not in _SPIN:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN["per_ms"] = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(ms * _SPIN["per_ms"]))


def time_apply(packed, bits, scale, zero, group, s_x, s_g, si, so, d_out, d_in, batch, reps=20):
    """Mean time of one kq_apply_quantized call and of its product kernel (event
    hook), over `reps` calls after warm-up; inputs resident on the device, the
    calls queued ahead of the GPU (hold_gpu)."""
    import torch

    import post_weight_quantization_amd as kq
    from post_weight_quantization_amd import _native as N

    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(batch)
    x = torch.randn(batch, d_in, device="cuda", generator=g)
    y = torch.empty(batch, d_out, device="cuda")
    ws = torch.empty(kq.kq_workspace_size(N.KQ_OP_APPLY_QUANTIZED, d_out, d_in, batch),
                     dtype=torch.uint8, device="cuda")
    call = lambda: kq.kq_apply_quantized(packed, bits, scale, zero, group, s_x, s_g, si, so, x, y=y, ws=ws)
    for _ in range(3):
        call()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    torch.cuda.synchronize()
    for k in range(reps):
        hold_gpu()
        ev[k][0].record(stream)
        kq.kq_set_kernel_events(N.KQ_OP_APPLY_QUANTIZED, ev[k][1], ev[k][2], stream)
        call()
        ev[k][3].record(stream)
    kq.kq_set_kernel_events(N.KQ_OP_APPLY_QUANTIZED)
    torch.cuda.synchronize()
    call_us = float(np.mean([e[0].elapsed_time(e[3]) for e in ev])) * 1e3
    kern_us = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    return call_us, kern_us


def time_apply_a4(packed, scale, zero, s_x, s_g, si, so, d_out, d_in, batch, clip=0.9, reps=20):
    """Mean time of one kq_apply_quantized_a4 call and of its product launches
    (event hook: every 16-vector launch of the call), inputs resident, the
    calls queued ahead of the GPU (hold_gpu)."""
    import torch

    import post_weight_quantization_amd as kq
    from post_weight_quantization_amd import _native as N

    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(batch)
    x = torch.randn(batch, d_in, device="cuda", generator=g)
    y = torch.empty(batch, d_out, device="cuda")
    ws = torch.empty(kq.kq_workspace_size(N.KQ_OP_APPLY_QUANTIZED_A4, d_out, d_in, batch),
                     dtype=torch.uint8, device="cuda")
    call = lambda: kq.kq_apply_quantized_a4(packed, scale, zero, s_x, s_g, si, so, x, clip, y=y, ws=ws)
    for _ in range(3):
        call()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    torch.cuda.synchronize()
    for k in range(reps):
        hold_gpu()
        ev[k][0].record(stream)
        kq.kq_set_kernel_events(N.KQ_OP_APPLY_QUANTIZED_A4, ev[k][1], ev[k][2], stream)
        call()
        ev[k][3].record(stream)
    kq.kq_set_kernel_events(N.KQ_OP_APPLY_QUANTIZED_A4)
    torch.cuda.synchronize()
    call_us = float(np.mean([e[0].elapsed_time(e[3]) for e in ev])) * 1e3
    kern_us = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    return call_us, kern_us


def run_inference(spec, codes, scale, zero, s_x, s_g, si, so):
    """Inference with the quantized layer (packed codes, y = S_G^-1 U^T W^' V
    S_X^-1 x): the layer this step quantized, and the 8192 x 28672 2-bit
    down_proj shape of the 70B workload with random codes. Bytes per product
    launch: packed codes + grids + the transformed input read + y1 written."""
    import torch

    import post_weight_quantization_amd as kq

    out = {}
    cases = [("layer", spec.d_out, spec.d_in, spec.bits, spec.group, codes, scale, zero, s_x, s_g, si, so)]
    m, n, b = 8192, 28672, 2
    g = torch.Generator(device="cuda").manual_seed(70)
    cases.append(("down_proj_8192x28672", m, n, b, 0,
                  torch.randint(0, 1 << b, (m, n), dtype=torch.uint8, device="cuda", generator=g),
                  torch.rand(m, 1, device="cuda", generator=g) * 0.01 + 0.005,
                  torch.randint(0, 1 << b, (m, 1), device="cuda", generator=g).float(),
                  torch.rand(n, device="cuda", generator=g) + 0.5,
                  torch.rand(m, device="cuda", generator=g) + 0.5,
                  (torch.randint(0, 2, (n,), device="cuda", generator=g) * 2 - 1).to(torch.int8),
                  (torch.randint(0, 2, (m,), device="cuda", generator=g) * 2 - 1).to(torch.int8)))
    for name, d_out, d_in, bits, group, cd, sc, zr, sx, sg, sgi, sgo in cases:
        packed = kq.kq_pack_codes(cd, bits)
        ng = d_in // group if group else 1
        rec = {"d_out": d_out, "d_in": d_in, "bits": bits, "group": group}
        for batch in (1, 4):
            call_us, kern_us = time_apply(packed, bits, sc, zr, group, sx, sg, sgi, sgo, d_out, d_in, batch)
            nbytes = packed.numel() * 4 + 8 * d_out * ng + 4 * batch * (d_in + d_out)
            rec[f"b{batch}"] = {"call_us": round(call_us, 2), "product_us": round(kern_us, 2),
                                "product_gbs": round(nbytes / kern_us / 1e3, 1),
                                "product_hbm_frac": round(nbytes / kern_us / 1e3 / (PEAK_HBM / 1e9), 4)}
        if bits == 2 and group == 0 and d_in % 512 == 0:
            # 4-bit activations: one product launch for the batch, the codes
            # and grids read once; per vector its d_in code bytes read and
            # its d_out fp32 outputs written
            a4 = {}
            for batch in (1, 16, 64, 256):
                call_us, kern_us = time_apply_a4(packed, sc.reshape(-1), zr.reshape(-1), sx, sg, sgi, sgo,
                                                 d_out, d_in, batch)
                nbytes = packed.numel() * 4 + 8 * d_out + batch * (d_in + 4 * d_out)
                a4[f"b{batch}"] = {"call_us": round(call_us, 2), "product_us": round(kern_us, 2),
                                   "product_gbs": round(nbytes / kern_us / 1e3, 1),
                                   "product_hbm_frac": round(nbytes / kern_us / 1e3 / (PEAK_HBM / 1e9), 4),
                                   "tops": round(2 * d_out * d_in * batch / kern_us / 1e6, 2)}
            rec["a4"] = a4
        out[name] = rec
    return out


def measure_peaks(reps=3):
    """The part's own ceilings, measured here (hand-written microbenchmarks in
    libkq_peaks.so): HBM read-only stream over 4 GiB, copy of 2 GiB, and
    back-to-back bf16 and fp32 MFMAs on every SIMD. Best of `reps` runs."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "post_weight_quantization_amd", "libkq_peaks.so"))
    for f in (lib.kqp_read, lib.kqp_copy, lib.kqp_mfma_bf16, lib.kqp_mfma_f32):
        f.restype = ctypes.c_int
    lib.kqp_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.kqp_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    for f in (lib.kqp_mfma_bf16, lib.kqp_mfma_f32):
        f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.empty(1024, dtype=torch.uint8, device="cuda")
    nb = 4 << 30
    buf = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty(nb // 8, dtype=torch.float32, device="cuda")

    def best(call, units):
        t = []
        for _ in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = call()
            b.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"peak microbenchmark failed: HIP error {rc}")
            t.append(a.elapsed_time(b))
        return units / (min(t[1:]) * 1e-3)

    read = best(lambda: lib.kqp_read(ctypes.c_void_p(buf.data_ptr()), nb, ctypes.c_void_p(sink.data_ptr()), sp), nb)
    half = nb // 2
    copy = best(lambda: lib.kqp_copy(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(dst.data_ptr()), half, sp),
                2 * half)
    del buf, dst
    blocks, it_b, it_f = 1024, 50000, 40000
    bf16 = best(lambda: lib.kqp_mfma_bf16(blocks, it_b, 0.0078125, ctypes.c_void_p(sink.data_ptr()), sp),
                blocks * 4 * 8 * it_b * 32768.0)
    f32 = best(lambda: lib.kqp_mfma_f32(blocks, it_f, 0.0078125, ctypes.c_void_p(sink.data_ptr()), sp),
               blocks * 4 * 8 * it_f * 4096.0)
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": round(read / 1e9, 1), "hbm_copy_gbs": round(copy / 1e9, 1),
            "bf16_mfma_tflops": round(bf16 / 1e12, 1), "fp32_mfma_tflops": round(f32 / 1e12, 2),
            "spec": {"hbm_gbs": PEAK_HBM / 1e9, "bf16_mfma_tflops": PEAK_BF16 / 1e12,
                     "fp32_mfma_tflops": PEAK_FP32_MFMA / 1e12},
            "how": "read: 4 GiB once; copy: 2 GiB read + 2 GiB written; MFMA: 1024 workgroups of 4 waves, "
                   "8 independent accumulators per wave, register operands; best of 3 timed runs"}


def summarize(spec, g):
    """Per-stage times, rates and fractions of one leg (published and measured peaks)."""
    costs = stage_costs(spec)
    st = g["stage_ms"]
    stages = {
        "cov_ms": round(st["cov"], 3),
        "cov_tflops": round(costs["cov_flops"] / st["cov"] / 1e9, 1),
        "biip_ms": round(st["biip"], 3),
        "biip_gbs": round(costs["biip_bytes"] / st["biip"] / 1e6, 1),
        "sens_ms": round(st["sens"], 3),
        "chol_ms": round(st["chol"], 3),
        "chol_tflops": round(costs["chol_flops"] / st["chol"] / 1e9, 2),
        "gptaq_ms": round(st["gptaq"], 3),
        "gptaq_tflops": round(costs["solve_flops"] / st["gptaq"] / 1e9, 2),
        "no_cov_ms": round(sum(v for k, v in st.items() if k != "cov"), 3),
    }
    stages["cov_frac_bf16"] = round(costs["cov_flops"] / (st["cov"] * 1e-3) / PEAK_BF16, 4)
    stages["biip_frac_hbm"] = round(costs["biip_bytes"] / (st["biip"] * 1e-3) / PEAK_HBM, 4)
    stages["biip_frac_hbm_read_once"] = round(costs["biip_min_bytes"] / (st["biip"] * 1e-3) / PEAK_HBM, 4)
    stages["chol_frac_fp32"] = round(costs["chol_flops"] / (st["chol"] * 1e-3) / PEAK_FP32_MFMA, 4)
    stages["gptaq_frac_fp32"] = round(costs["solve_flops"] / (st["gptaq"] * 1e-3) / PEAK_FP32_MFMA, 4)
    cov_ms = g["cov_kernel_ms"]
    cov_tf = costs["cov_flops"] / (cov_ms * 1e-3)
    cov_kernel = {"kernel": "cov_bf16_kernel", "kernel_ms": round(cov_ms, 4),
                  "achieved": round(cov_tf / 1e12, 2), "frac": round(cov_tf / PEAK_BF16, 4)}
    trailing = None
    if g["trail_kernel_ms"]:
        # the sweep's largest lazy GEMM: d_out x (d_in - 512) x 512, event-timed
        tf = 2.0 * spec.d_out * (spec.d_in - 512) * 512
        tms = g["trail_kernel_ms"]
        # the library runs fp32 products with at least 200 tiles of 128 x 128
        # (and no triangular operand) on the bf16 matrix cores, as six
        # products of three-term bf16 splits; fewer tiles on the fp32 kernel
        x3 = -(-spec.d_out // 128) * -(-(spec.d_in - 512) // 128) >= 200
        trailing = {"kernel": ("gemm_x3_kernel (fp32 on three bf16 terms)" if x3 else "gemm_f32_kernel")
                    + ", first superblock's trailing update",
                    "shape": [spec.d_out, spec.d_in - 512, 512], "kernel_ms": round(tms, 4),
                    "achieved": round(tf / (tms * 1e-3) / 1e12, 2), "peak": PEAK_FP32_MFMA / 1e12,
                    "unit": "TFLOP/s", "frac": round(tf / (tms * 1e-3) / PEAK_FP32_MFMA, 4)}
        if x3:
            # what the matrix cores executed: six bf16 products per fp32 one
            trailing["bf16_mfma_frac"] = round(6 * tf / (tms * 1e-3) / PEAK_BF16, 4)
    return costs, stages, cov_kernel, trailing


def with_measured(stages, cov_kernel, trailing, peaks):
    """Fractions of the measured ceilings beside the published ones."""
    if not peaks:
        return
    stages["cov_frac_measured_bf16"] = round(stages["cov_tflops"] / peaks["bf16_mfma_tflops"], 4)
    stages["biip_frac_measured_copy"] = round(stages["biip_gbs"] / peaks["hbm_copy_gbs"], 4)
    stages["chol_frac_measured_fp32"] = round(stages["chol_tflops"] / peaks["fp32_mfma_tflops"], 4)
    stages["gptaq_frac_measured_fp32"] = round(stages["gptaq_tflops"] / peaks["fp32_mfma_tflops"], 4)
    cov_kernel["frac_measured"] = round(cov_kernel["achieved"] / peaks["bf16_mfma_tflops"], 4)
    if trailing:
        trailing["frac_measured"] = round(trailing["achieved"] / peaks["fp32_mfma_tflops"], 4)


def run_second_leg(workload, layer, steps, warmup, peaks, cpu_prefix=0):
    """The whole path on a second layer shape (default: the LLaMA-3-70B
    down_proj, W 8192 x 28672, 131072 bf16 tokens, 2-bit per channel),
    device-resident inputs from the same generator, timed per stage. With
    cpu_prefix > 0 the oracle is timed per stage on the same inputs
    (covariances over that token prefix, scaled; the rest at full size,
    several minutes of host time at this shape)."""
    import torch

    from synth import WORKLOADS, layer_specs, make_layer

    torch.cuda.empty_cache()
    spec = layer_specs(WORKLOADS[workload])[layer]
    t0 = time.perf_counter()
    data = make_layer(spec)
    print(f"[bench] generated {spec.name} {spec.d_out}x{spec.d_in}, N={spec.n_tok} "
          f"in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    g = run_gpu(spec, steps, warmup, data, extras=False)
    torch.cuda.empty_cache()
    cpu = None
    if cpu_prefix:
        cpu = cpu_baseline(spec, data, min(cpu_prefix, spec.n_tok))
        print(f"[bench] {spec.name} cpu oracle stages (s): {json.dumps(cpu['stages_s'])}", file=sys.stderr,
              flush=True)
    del data
    print(f"[bench] {spec.name} gpu stages (ms): {json.dumps(g['stage_ms'])}", file=sys.stderr, flush=True)
    _, stages, cov_kernel, trailing = summarize(spec, g)
    with_measured(stages, cov_kernel, trailing, peaks)
    return {"workload": f"{workload}: {spec.name} W {spec.d_out}x{spec.d_in}, {spec.n_tok} {spec.dtype} "
                        f"tokens, {spec.bits}-bit {'per-channel' if not spec.group else f'group {spec.group}'}",
            "steps": steps, "warmup": warmup, "ms_per_layer": round(g["wall_s"] * 1e3 / steps, 3),
            "stages": stages, "cov_kernel": cov_kernel, "trailing_gemm": trailing,
            "sensitivity": g["sens"][2], "objective": g["obj"], "objective_rtn": g["obj_rtn"],
            "cpu_oracle": cpu}


def copy_calibration(mib):
    """One plain device-to-device copy of `mib` MiB (reads and writes that many bytes)."""
    import torch

    a = torch.ones(mib << 18, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {mib} MiB read + {mib} MiB written", file=sys.stderr, flush=True)
    del a, b


def cpu_baseline(spec, data, prefix):
    """The oracle as it stands, on a bounded sample: covariances over a token
    prefix (scaled to the full token count), every later stage at full size."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t = {}
    t0 = time.perf_counter()
    HX, D, HG = oracle.covariances(data["x"][:prefix], data["xq"][:prefix], data["g"][:prefix])
    t["cov_prefix"] = time.perf_counter() - t0
    print(f"[bench] oracle covariances over {prefix} tokens: {t['cov_prefix']:.1f} s", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    W2, HX2, D2, HG2, _, _ = oracle.biip(data["W"], HX, D, HG, data["sign_in"], data["sign_out"])
    t["biip"] = time.perf_counter() - t0
    print(f"[bench] oracle BiIP: {t['biip']:.1f} s", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    oracle.sensitivity(HX2, HG2)
    U = oracle.inv_factor(HX2, spec.damp)
    t["chol"] = time.perf_counter() - t0
    print(f"[bench] oracle factor: {t['chol']:.1f} s", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    P = oracle.form_p(D2, U)
    oracle.sweep(W2, U, P, spec.bits, spec.group, spec.block)
    t["gptaq"] = time.perf_counter() - t0
    est = t["cov_prefix"] * spec.n_tok / prefix + t["biip"] + t["chol"] + t["gptaq"]
    sample = (f"covariances over the first {prefix} of {spec.n_tok} tokens, time scaled x"
              f"{spec.n_tok // prefix}; BiIP, factor, P and sweep at full size "
              f"(measured {sum(t.values()):.1f} s)")
    return dict(value=est * 1e3, unit="ms", cores=int(cores), nproc=os.cpu_count(), kind="oracle",
                sample=sample,
                stages_s={k: round(v, 3) for k, v in t.items()})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama2-7b-q_proj")
    ap.add_argument("--layer", type=int, default=0, help="sublayer index within the workload")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-prefix", type=int, default=4096)
    ap.add_argument("--no-peaks", action="store_true", help="skip the on-box peak microbenchmarks")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the legs after the layer step (inference, output feedback, streaming)")
    ap.add_argument("--second", default="llama3-70b-q-down:1", metavar="WORKLOAD:LAYER",
                    help="a second layer timed per stage after the main one ('none' to skip)")
    ap.add_argument("--second-steps", type=int, default=2)
    ap.add_argument("--cpu-second-prefix", type=int, default=0, metavar="TOKENS",
                    help="also time the oracle per stage on the second layer (covariances over this "
                         "many tokens, scaled); 0 skips it")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this solver's path runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from synth import WORKLOADS, layer_specs, make_layer

    spec = layer_specs(WORKLOADS[args.workload])[args.layer]
    t0 = time.perf_counter()
    data = make_layer(spec)
    print(f"[bench] generated {spec.name} {spec.d_out}x{spec.d_in}, N={spec.n_tok} "
          f"in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    if args.copy_calib:
        copy_calibration(args.copy_calib)
    g = run_gpu(spec, args.steps, args.warmup, data, extras=not args.no_extras)
    print(f"[bench] gpu stages (ms): {json.dumps(g['stage_ms'])}", file=sys.stderr, flush=True)
    costs, stages, cov_kernel, trailing = summarize(spec, g)
    ms = g["wall_s"] * 1e3 / args.steps
    cov_ms = g["cov_kernel_ms"]
    achieved = costs["cov_flops"] / (cov_ms * 1e-3)
    src = open(os.path.join(ROOT, "post_weight_quantization_amd", "csrc", "cov.hip"), "rb").read()
    traffic = None
    if (COV_TRAFFIC["cov_sha256"] == hashlib.sha256(src).hexdigest()
            and (spec.d_out, spec.d_in, spec.n_tok) == (4096, 4096, 131072)):
        traffic = COV_TRAFFIC["bytes"]
    roof = {"kernel": "cov_bf16_kernel", "kernel_ms": round(cov_ms, 4), "bound": "mfma",
            "achieved": round(achieved / 1e12, 2), "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16, 4), "traffic": traffic}
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks()
        print(f"[bench] measured peaks: {json.dumps(peaks)}", file=sys.stderr, flush=True)
        roof["peak_measured"] = peaks["bf16_mfma_tflops"]
        roof["frac_measured"] = round(achieved / 1e12 / peaks["bf16_mfma_tflops"], 4)
    with_measured(stages, cov_kernel, trailing, peaks)
    second = None
    if args.second and args.second != "none":
        wl, _, li = args.second.partition(":")
        second = run_second_leg(wl, int(li or 0), args.second_steps, 1, peaks, args.cpu_second_prefix)
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(spec, data, min(args.cpu_prefix, spec.n_tok))
        print(f"[bench] cpu oracle stages (s): {json.dumps(cpu['stages_s'])}", file=sys.stderr, flush=True)
        cpu.pop("stages_s")
    out = {
        "metric": "KronQ layer-quant ms at 4096x4096 2-bit; SYRK/trailing-GEMM MFMA %",
        "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {spec.name} W {spec.d_out}x{spec.d_in}, "
                               f"{spec.n_tok} {spec.dtype} tokens, {spec.bits}-bit "
                               f"{'per-channel' if not spec.group else f'group {spec.group}'}",
                   "d_out": spec.d_out, "d_in": spec.d_in, "n_tok": spec.n_tok,
                   "inputs": spec.dtype, "bits": spec.bits, "group": spec.group,
                   "block": spec.block, "damp": spec.damp},
        "roofline": roof,
        "measured_peaks": peaks,
        "trailing_gemm": trailing,
        "stages": stages,
        "sensitivity": g["sens"][2],
        "objective": g["obj"], "objective_rtn": g["obj_rtn"],
        "cpu_baseline": cpu,
        "inference": g["inference"],
        "streaming_covariances": g["streaming"],
        "output_feedback": g["output_feedback"],
        "second_layer": second,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
