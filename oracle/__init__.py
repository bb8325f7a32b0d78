"""CPU oracle (float64 NumPy) for Beam 1.0 hybrid GQA attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline leg of bench.py; never by the product path.
"""
from .beam_attention import *  # noqa: F401,F403
from .beam_attention import Config, LOCAL, GLOBAL  # noqa: F401
from . import router  # noqa: F401
from . import projection  # noqa: F401
