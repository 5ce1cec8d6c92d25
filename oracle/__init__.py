"""CPU oracle (float64 numpy) for the latent-MoE block — test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg import this
package; the HIP library never does.
"""
from .lmoe_oracle import (BF16_MAX, E2M1_VALUES, Layer, bf16_to_f64, block_forward, decode, e4m3_decode,  # noqa: F401
                          expert_matrices, mxfp4_decode, nvfp4_decode, permute, rmsnorm, round_to_bf16, route, silu,
                          stack_step, swiglu)
