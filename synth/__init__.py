"""Seeded synthetic workloads for the MoE layer (inputs only).

Holds the five layer shapes and the seeded random draws of their inputs and
master weights.  It contains none of the layer's arithmetic: no routing, no
quantization, no contraction.  Both the HIP path's tests/bench and the CPU
oracle take their inputs from here.
"""

from .workloads import *  # noqa: F401,F403
