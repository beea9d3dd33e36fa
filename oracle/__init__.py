"""fp64 CPU oracle of the sampling-transform scoring core (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this package; the HIP library never does.
"""
from .stce_oracle import (  # noqa: F401
    E4M3_MAX, MARGIN, backward, e4m3_decode, e4m3_encode, fp8_dequant_rows, fp8_dequant_weight, fp8_logits, fp8_quantize_rows,
    backward_pre_gemm, bf16_lane_keys, binding_filters, canonical_f32, chunk_logits, dlogits,
    forward, gradient_products, in_support,
    OBJECTIVES, order_keys, order_row, policy_loss, pre_gemm_hidden, round_to_bf16, sample_targets,
    scale_logits, support, support_row,
)
