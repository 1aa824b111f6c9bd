"""CPU oracle for group-wise asymmetric int4 weight-only quantization, its
fake-quantize round trip, the pre-shuffled weight layout, the W4A16
linear layer, the W4A8 path (per-token int8 activations), and int8
weight-only quantization with its linear.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check and the CPU
baseline leg of the benchmark use it. It shares no code with the HIP
library and imports nothing from it.
"""
from .ref import (  # noqa: F401
    GROUP_SIZES,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    quantize_ref,
    unpack_codes_ref,
    repack_preshuffled_ref,
    dequant_ref,
    fake_quant_ref,
    linear_ref,
    linear_rows_ref,
    act_quant_ref,
    quantize_int8_ref,
    linear_int8_ref,
    w4a8_linear_ref,
    rel_frobenius,
)
