"""fp64 CPU oracle for fused linear cross-entropy (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library.
"""
from .flce_ref import (IGNORE_INDEX, REDUCTIONS, CEResult, ORPOResult, Result, ResultEx,
                       cross_entropy, dW_rows, dX_rows, flce, flce_ex, forward_rows, loss_blocked,
                       orpo, orpo_rows, PAIR_KINDS, PreferenceResult, preference, KTOResult, kto,
                       kto_reference_point)

__all__ = ["IGNORE_INDEX", "REDUCTIONS", "CEResult", "ORPOResult", "Result", "ResultEx",
           "cross_entropy", "flce", "flce_ex", "orpo", "orpo_rows", "PAIR_KINDS",
           "PreferenceResult", "preference", "KTOResult", "kto", "kto_reference_point",
           "forward_rows", "loss_blocked", "dX_rows", "dW_rows"]
