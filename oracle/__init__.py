"""Float64 CPU oracle for the S5 forward path.

Test infrastructure only: imported by tests/, by the package smoke check and
by the benchmark's CPU-baseline leg, never by the library itself.
"""
from . import s5_oracle  # noqa: F401
