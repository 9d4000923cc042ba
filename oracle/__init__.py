"""CPU oracle of the MoE expert path - test infrastructure only.

Only tests/, the smoke check in __graft_entry__.py and the CPU-baseline leg of
bench.py may import this package.  The HIP library never does.
"""
from . import moe_oracle  # noqa: F401
from .moe_oracle import (gate, permute, grouped_ffn, combine, stats, moe_layer,  # noqa: F401
                         assignment_groups, expert_of_group, to_f64, bf16_bits_to_f64,
                         f64_to_bf16_bits, silu_product)
