"""Float64 CPU oracle for ragged grouped-query attention (forward + full VJP).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path.
"""
from . import dropout
from .attention import forward, rows_vjp, sequence_vjp, vjp, window_bounds

__all__ = ["forward", "vjp", "sequence_vjp", "rows_vjp", "window_bounds", "dropout"]
