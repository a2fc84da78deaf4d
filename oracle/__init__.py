"""Double-precision CPU oracle for row-wise LayerNorm / RMSNorm, a norm feeding a linear
projection, and attention over normalised queries and keys (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package. The HIP library never does.
"""
from .oracle import (BF16, BF16_F32W, F16, F16_F32W, F32, LAYERNORM, NO_NORM,  # noqa: F401
                     RMSNORM, Oracle, act_dtype, weight_dtype, bwd, decode, default, fwd,
                     norm_attention, norm_linear, num_threads, round_bf16, round_f16,
                     set_num_threads)
