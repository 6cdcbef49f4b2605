"""CPU oracle for the MoE expert feed-forward layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
it is used by tests/, by __graft_entry__.smoke() to check one small call, and
by bench.py's cpu_baseline leg. It shares no code with the HIP library and
does not import it.

Plain numpy in float64, one expert at a time, in the shape of the Hugging
Face per-expert loop shown in "Efficient MoE Training for Biological
Foundation Models", Challenge 1: Fragmented expert kernels.
"""
from .moe_oracle import *  # noqa: F401,F403
from .mxfp8 import *  # noqa: F401,F403
from .router import *  # noqa: F401,F403
from .fp8_tensor import *  # noqa: F401,F403
