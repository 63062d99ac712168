"""CPU oracle for GPTQ layer-wise weight quantization.

TEST INFRASTRUCTURE ONLY.  This package is imported by the tests, by the smoke
check in __graft_entry__ and by the CPU-baseline leg of bench.py.  The GPU
library (post_weight_quantization_24_amd) never imports, links or calls it, and
this package imports nothing from there: the two share no code.

Parity status of every function is stated in gptq_oracle's header.
"""

from .gptq_oracle import *  # noqa: F401,F403
