"""Plain fp64 CPU reference ("oracle") of the MSA hot path.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library or its binding.  It
shares no code with the GPU path.  The C source (``msa_oracle.c``) documents
each definition and the page/section it follows.
"""
from .oracle import *  # noqa: F401,F403
