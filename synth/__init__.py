"""Seeded synthetic inputs for the paged-KV decode path.

This package only draws random numbers and lays out workload shapes: sequence
lengths, the order in which physical blocks are handed out, branch suffix
lengths, which blocks get offloaded, and the values of Q, K and V. It holds none
of the method's arithmetic (no address translation, no slot computation, no
attention), so both the library under test and the CPU oracle can take their
inputs from here without sharing any of the computation they are compared on.
"""

from .configs import CONFIGS, Workload, get_config  # noqa: F401
from . import gen  # noqa: F401
