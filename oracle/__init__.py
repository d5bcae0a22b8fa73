"""CPU oracle for the sparse MoE layer, forward and backward (test
infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark use
this package; the HIP library never imports, links or calls it.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle_backward import *  # noqa: F401,F403
