"""Oracle for the DM0-style dual-expert merged-attention path.

TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct CPU implementation (numpy, float64
unless a function says otherwise) used to check the HIP library.  Only the test-suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the library never does.
It shares no code with the HIP path: it imports neither the package nor its binding.
"""
from .dm_oracle import *  # noqa: F401,F403
