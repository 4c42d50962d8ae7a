"""fp64 CPU oracle for piecewise block-sparse attention.

Test infrastructure only: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product path.
"""
from .pisa_oracle import MODE_APPROX, MODE_DROP, attention, precompute, route, route_scores

__all__ = ["MODE_APPROX", "MODE_DROP", "attention", "precompute", "route", "route_scores"]
