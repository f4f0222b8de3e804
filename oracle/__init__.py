"""CPU oracle (TEST INFRASTRUCTURE ONLY): a plain, slow, float64 NumPy implementation of oracle
top-k selection and sparse/dense decode attention, and (oracle/sketch.py) of the reduced-byte
indexer that ranks an int8 sketch of the keys and re-ranks its candidates exactly.  Only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may import it; the HIP library
never does, and the two share no code.

Every function is pinned by the CPU tests (tests/test_oracle_pins.py, tests/test_sketch_oracle.py)
against exact rational arithmetic, brute force over all subsets of tiny inputs, closed forms,
SciPy routines and invariants.  The pages print no worked example with values, so no pin
compares against a number quoted from them."""

from .reference import *  # noqa: F401,F403
from .reference import __all__ as _ref_all
from .sketch import *  # noqa: F401,F403
from .sketch import __all__ as _sketch_all

__all__ = list(_ref_all) + list(_sketch_all)
