"""CPU oracle for queues of small tensor ops.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the runtime package.
It is a plain op-by-op interpreter (numpy, fp64 for reductions and
transcendentals) that shares no code with the HIP path.

Pinned functions (see ``tests/test_oracle_pins.py``): every op kind of
``interpreter.apply_op``, the bf16 conversions and ``compare``.  Parity
unpinned: the decode workload as a whole (no page defines a layer's math; it is
pinned only through its individual ops) and GPUOS's own scheduling semantics
(the pages give none beyond "run the queued ops").
"""

from .interpreter import (EXACT_KINDS, TOL_KINDS, OracleError, WeightCache, apply_op,
                          bf16_to_f32, f32_to_bf16, local_check, out_len, run)
from .compare import RTOL, EndToEnd, Mismatch, compare, end_to_end

__all__ = ["EXACT_KINDS", "TOL_KINDS", "OracleError", "WeightCache", "apply_op", "bf16_to_f32",
           "f32_to_bf16", "local_check", "out_len", "run", "RTOL", "EndToEnd", "Mismatch",
           "compare", "end_to_end"]
