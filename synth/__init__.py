"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package only draws random tensors and describes workload shapes.  It holds
none of the attention arithmetic, none of the position or mask rules and none of
the merge rules: those live, independently, in ``oracle/`` and in the HIP
library.
"""
from .configs import CONFIGS, Config, get  # noqa: F401
from .gen import normal_draw, make_dense_case, make_ring_case  # noqa: F401
