"""fp64 CPU oracle for coverage-rule sparse paged decode attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
imports nothing from the product package.
"""
from .moira_oracle import *  # noqa: F401,F403
from .moira_oracle import __all__  # noqa: F401
