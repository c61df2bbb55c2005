"""The parity comparators live with the oracle (oracle/tolerances.py), where
the benchmark's CPU-baseline leg can use them too; the tests import them from
here."""
from oracle.tolerances import (FLOOR_FACTOR, assert_close, assert_close_bounded, assert_reduction_close,  # noqa: F401
                               compare, from_storage, to_storage, ulp, values)
