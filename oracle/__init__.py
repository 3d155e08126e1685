"""Float64 CPU oracle for the q4g64 weight-only matmul (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it.
"""

from .q4g64 import (  # noqa: F401
    BITS,
    activations_f64,
    bf16_to_f64,
    dequantize,
    error_weight,
    matmul_rows,
    matmul_rows_exact,
    matmul_rows_fraction,
    silu,
    swiglu,
    unpack_codes,
    words_per_row,
)
from .fp8block import (  # noqa: F401
    dequantize_fp8,
    e4m3_to_f64,
    error_weight_fp8,
    matmul_rows_fp8,
    matmul_rows_fp8_exact,
    matmul_rows_fp8_fraction,
)
from .rope_kv import attention_gate, rms_norm, rope, rope_angles, rope_kv  # noqa: F401,E402
