"""Oracle package: a plain, slow CPU statement of the MoE-layer forward pass,
of its backward pass (``oracle.moe_backward``) and of token condensation
(``oracle.condense``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
from . import condense  # noqa: F401
from . import moe_backward  # noqa: F401
