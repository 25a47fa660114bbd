"""CPU oracle for the Prox two-stage sparse SwiGLU FFN step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It is independent of
the HIP library: the two share no code, and neither imports the other.
"""
from .prox_oracle import (Layer, build, calibrate_sequential, dense,  # noqa: F401
                          dequantize, forward, forward_batch, forward_ts, gate_act,
                          input_mask,
                          lower_quantile, proxy, quantize, rmsnorm, round_bf16,
                          stack_forward, stack_forward_ts, stage2, threshold_mask, topk)
