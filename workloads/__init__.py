"""Seeded synthetic workloads for the speculative-verify Gated DeltaNet route.

This package only draws inputs: tensor shapes, random values and tree / slot /
acceptance structure.  It holds none of the route's arithmetic, so both the
HIP path and the CPU oracle can consume the same arrays without sharing code.
"""

from .gen import (  # noqa: F401
    EDGE_KINDS,
    WORKLOADS,
    Workload,
    layer_params,
    round_inputs,
    round_structure,
    path_to_root,
    synth_case,
    edge_case,
)
