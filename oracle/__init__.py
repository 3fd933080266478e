"""CPU oracle for the MoE routing + expert-FFN path (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package
entry file and the CPU-baseline leg of the benchmark may import it.  The
product path (the HIP library and its Python binding) never imports, links or
calls anything here, and this package imports nothing from the product path.
"""
from .moe_oracle import *  # noqa: F401,F403
