"""Seeded synthetic inputs for the q4g64 weight-only matmul.

This package is the only code that both the float64 oracle (``oracle/``) and the
GPU path consume. It draws random numbers and stores them in the canonical
input format; it performs none of the method's arithmetic (no unpacking, no
dequantization, no dot products).
"""

from .workloads import (  # noqa: F401
    CONFIG_NAMES,
    FP8Weight,
    QWeight,
    bf16_bits_from_f64,
    concat_rows,
    config,
    draw_bf16_rows,
    draw_f32_rows,
    draw_fp8_weight,
    draw_qweight,
    pack_codes_bits,
    pack_codes_low_nibble_first,
    sha256_of,
)
