"""CPU oracle for the MLA decode step.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and
the benchmark's CPU-baseline leg, never by the GPU library.  It shares no
code with the library; both read the seeded inputs from ``mla_synth``.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, printed values of the pages (``tests/golden/``), invariants,
special cases with known answers and a scalar brute force.  No function is
parity-unpinned.
"""
from . import mla_oracle, absorbed_fp64, brute, closed_forms  # noqa: F401
from .mla_oracle import (  # noqa: F401
    attend_sequence,
    decode,
    default_scale,
    latent_rows,
    rope_inv_freq,
    rope_rotate,
    softmax,
)
