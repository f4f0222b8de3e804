"""CPU oracle (TEST INFRASTRUCTURE ONLY): a plain, slow, float64 NumPy implementation of oracle
top-k selection and sparse/dense decode attention.  Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the HIP library never does, and the two share
no code.

Every function is pinned by the CPU tests (tests/test_oracle_pins.py) against exact rational
arithmetic, brute force over all subsets of tiny inputs, closed forms, SciPy routines and
invariants.  The pages print no worked example with values, so no pin compares against a number
quoted from them."""

from .reference import *  # noqa: F401,F403
from .reference import __all__  # noqa: F401
