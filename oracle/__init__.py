"""fp64 CPU oracle for causal linear attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the HIP library.
"""
from .oracle import (BETA_MAPS, GATE_MAPS, GATES, QK_MAPS, RULES, OracleLib,  # noqa: F401
                     build, decode_step, default, deltaproduct, deltaproduct_bwd, max_threads, normalized,
                     prepare_beta, prepare_gate, prepare_qk, recurrence, recurrence_bwd)
