"""CPU oracle for Prism dynamic sparse video self-attention.

TEST INFRASTRUCTURE ONLY.  Plain, slow numpy written from the Prism pages;
it shares no code with the HIP library.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does.
"""

from .prism_oracle import *  # noqa: F401,F403
from .prism_oracle import __all__  # noqa: F401
