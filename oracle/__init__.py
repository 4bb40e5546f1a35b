"""Plain fp64 CPU oracle of KronQ's per-layer solver.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code with the native HIP library
(no kernels, headers, helpers, tables or pre/post-processing); the only thing
both sides read is the seeded input data from ``synth/``.

Every function is written from the pages' statement of the method (KronQ:
LLM Quantization via Kronecker-Factored Hessian, as summarised by hyper.ai and
gist.science) and cites the passage it follows. Where the pages leave a step
open, the reading taken is stated next to the code.

Parity pins: each function here is checked by ``tests/test_oracle_pins.py``
(``tests/test_oracle_yaqa.py`` for the rounding with output-side feedback)
against closed forms, brute force or library routines. One result is
"parity unpinned" beyond the oracle itself: the exact integer codes of the
full-size workloads, since the pages print no worked example.
"""
from . import deploy  # noqa: F401
from . import yaqa  # noqa: F401
from .kronq import (  # noqa: F401
    allocate_bits,
    apply_hadamard_left,
    apply_hadamard_right,
    bf16_rne,
    biip,
    biip_scales,
    covariance_diagonals,
    covariances,
    covariances_chunked,
    cv_in_out,
    damped,
    decode_inputs,
    form_p,
    form_p_rows,
    grid_fp32,
    hadamard_block,
    hadamard_rows,
    inv_factor,
    mu_incoherence,
    objective,
    quantize_layer,
    rtn,
    scaled_traces,
    sensitivity,
    solve_layer,
    sweep,
    sylvester,
)
