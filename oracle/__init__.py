"""fp64 CPU oracle for the int4 block-32 decode step (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  The product library never does.
"""
from . import vv_oracle  # noqa: F401
