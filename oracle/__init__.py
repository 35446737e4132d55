"""CPU oracle for the DeepSeek-V3.2-Exp MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything here: only the tests, the package entry's smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library.
"""
from .moe_oracle import *  # noqa: F401,F403
