"""CPU oracle for the exact-load rebalancing path (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU
baseline may import this package; the product path never does.
"""
from .ultraep_oracle import (Plan, balance, bf16_bits_to_f64, combine, combine_backward,  # noqa: F401
                             count, f64_to_bf16_bits, feasible, fold, layout, ordinals, permute,
                             plan, quota_grid, relay_plan, replica_slots, reroute, weight_sync, local_takes, reroute_local,
                             RELAY_ADAPTIVE, RELAY_DIRECT, RELAY_FORCE)
