"""CPU oracle for the span-commit / verify path — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 numpy implementation of what the path computes, written from the
pages (Copy-as-Decode §2.4 and Appendix K; SwitchSD's block-triangular verification
paragraph; the PLD page's n-gram match and verification scan).  It shares no code with
the HIP library and imports nothing from the `spec_verify_cad_amd` package.

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark may
import it.  The product path never calls it; there is no CPU fallback.
"""
from .cad_oracle import *  # noqa: F401,F403
