"""CPU oracle for the residue-compensated block-scaled FP4 linear layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the bench's
CPU-baseline leg, never by the product path.  It shares no code with the HIP
library; see ``rsfp4_oracle.c`` for the arithmetic and its sources.
"""
from .oracle import *  # noqa: F401,F403
