"""Seeded synthetic workloads for paged GQA decode attention.

This package only draws inputs: shapes, context lengths, the physical-block
placement permutation, the order of the setup operations, and N(0, 1) tensor
values rounded to the storage dtype.  It holds none of the method's
arithmetic, and both the HIP path's callers and the oracle's callers take
their inputs from it.
"""
from .configs import (CONFIGS, EXTEND_CONFIGS, EXTEND_SMALL, SMALL, WINDOW_CONFIGS, Workload,  # noqa: F401
                      custom_workload, history_rows_of, make_extend_workload, make_request_values, make_values,
                      make_window_workload, make_workload, setup_ops, shape_scores)
