"""CPU oracle (test infrastructure only): see ``nm_oracle``.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The HIP library never does.
"""
from . import nm_oracle  # noqa: F401
