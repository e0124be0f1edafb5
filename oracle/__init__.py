"""CPU fp64 oracle of the MoE feed-forward layer.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  The HIP path never imports it and it imports nothing
from the HIP path.
"""
from . import moe_oracle  # noqa: F401
