"""fp64 CPU oracle of the LOCKS decode hot path. Test infrastructure only:
imported by the tests, the entry module's smoke check and the benchmark's
CPU-baseline leg, never by the product library."""
from . import locks_oracle  # noqa: F401
