"""CPU oracle for the int8-state gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy implementation of what the GPU library computes.  Only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
library itself never does, and the two share no code.

Parity status of each function is listed in ``oracle.gdnq_oracle``'s header.
"""

from .gdnq_oracle import (  # noqa: F401
    quantize_rows,
    dequantize,
    wht_matrix,
    gdn_step,
    ssd_step,
    run_windowed,
    decode_step,
    round_bf16,
    round_e4m3,
    quantize_e4m3_vector,
    prefill,
    chunked_fp64,
    ssd_closed_form,
    sweep_mirror,
    gdn_transition,
    propagate_key,
    run_sliding,
    sliding_ring_slots,
    decode_step_sliding,
)
