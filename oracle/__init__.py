"""Double-precision CPU oracle for row-wise LayerNorm / RMSNorm (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package. The HIP library never does.
"""
from .oracle import (BF16, BF16_F32W, F32, LAYERNORM, RMSNORM, Oracle, act_dtype,  # noqa: F401
                     weight_dtype, bwd, decode, default,
                     fwd, num_threads, round_bf16, set_num_threads)
