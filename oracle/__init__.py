"""Float64 CPU oracle for speculative-sampling verification.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke entry point and
the benchmark's CPU-baseline leg, never by the product library.  See
``oracle.spec_oracle`` for the sources and the readings of the pages.
"""

from .spec_oracle import *  # noqa: F401,F403
from .spec_oracle import __all__  # noqa: F401
