"""CPU oracle for the MXFP8 W8A8 linear layer.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the CPU-baseline
leg of the bench are the only callers. The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and nothing
here imports the product package.

Everything is plain numpy in float64 (float32 where the pages fix FP32
scales). ``oracle/mx_oracle.py`` is the MXFP8 scheme, ``oracle/pc_oracle.py``
the per-output-channel FP8 scheme; each function cites the passage it follows.
"""

from .mx_oracle import (  # noqa: F401
    E4M3_MAX,
    E4M3_EMAX,
    E8M0_BIAS,
    GELU_SLOPE_MAX,
    GROUP,
    bf16_round,
    bf16_ulp,
    dequantize_mx,
    e4m3_decode,
    e4m3_encode,
    e8m0_decode,
    gelu_tanh,
    linear_ref,
    mx_scale_code,
    quantize_mx,
    tolerance,
)
from .pc_oracle import QMAX, dequantize_pc, linear_pc_ref, quantize_pc  # noqa: F401
