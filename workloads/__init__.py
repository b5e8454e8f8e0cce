"""Seeded synthetic workloads shared by the tests, the smoke check and the
benchmark.  Holds the workload shapes and the input generator only: none of
the layer's arithmetic (routing, permutation, expert maps, combine) lives here.
"""

from .gen import (CONFIGS, LayerConfig, make_inputs, make_exact_router_inputs,  # noqa: F401
                  oracle_view, spec_of)
