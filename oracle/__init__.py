"""CPU oracle for the exact-load rebalancing path (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU
baseline may import this package; the product path never does.
"""
from .ultraep_oracle import (Plan, balance, count, feasible, fold, layout, ordinals,  # noqa: F401
                             permute, plan, quota_grid, reroute)
