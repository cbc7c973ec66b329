"""fp64 CPU oracle for remapped-position RoPE attention (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package. The HIP library never does, and the oracle never imports the library.
"""
from .rope_attention import (  # noqa: F401
    MODES, rope_theta, rotate, periodic_index, group_size, remote_index, rope_apply_ref,
    continuous_scale, round_to_bf16, round_operand, prefill_ref, decode_ref, bifocal_eq7_ref,
    brute_force_prefill,
)
