"""fp64 CPU oracle for causal linear attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the HIP library.
"""
from .oracle import (GATES, RULES, OracleLib, build, decode_step, default,  # noqa: F401
                     deltaproduct, max_threads, recurrence)
