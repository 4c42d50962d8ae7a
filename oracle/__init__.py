"""fp64 CPU oracle for piecewise block-sparse attention.

Test infrastructure only: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product path.
"""
from .pisa_oracle import (MODE_APPROX, MODE_DROP, MODE_FIRST, MODE_ZEROTH, attention, precompute,
                          route, route_scores)

__all__ = ["MODE_APPROX", "MODE_DROP", "MODE_ZEROTH", "MODE_FIRST", "attention", "precompute",
           "route", "route_scores"]
