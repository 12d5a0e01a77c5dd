"""CPU oracle for three-tier activation-sparse decode (test infrastructure).

This package is test infrastructure only. Nothing on the product path imports
it: only the tests, the smoke check and the benchmark's CPU-baseline leg may
call it. It shares no code with the HIP library.
"""
from .spax_oracle import *  # noqa: F401,F403
from .spax_oracle import __all__  # noqa: F401
