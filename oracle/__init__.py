"""CPU oracle (float64 NumPy) for the KVA projector -- test infrastructure.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never does.
"""
from .ref import *  # noqa: F401,F403
from . import ref  # noqa: F401
