"""CPU oracle for the INT8 convrot linear layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the HIP product path never imports it.
"""
from .convrot_oracle import *  # noqa: F401,F403
from .convrot_oracle import (  # noqa: F401
    MAX_K_INT32,
    QMAX,
    check_group,
    dequantize,
    gelu,
    h4,
    int_gemm,
    int_gemm_int64,
    lora_correction,
    lora_down,
    lora_up,
    linear,
    log4_group,
    pack_activations,
    quantize_activation_rows,
    quantize_weight_rows,
    quantize_weights,
    reference_linear_fp64,
    rotate,
    rotation_matrix,
    round_bf16,
    round_half_away,
)
