"""CPU oracle for the 4-bit block-quantized MoE prefill layer.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The GPU library never calls into it, and it shares no code with the GPU
path: it reads the same packed bytes and recomputes everything from the
definition in float64 with numpy.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
