"""CPU oracle for parallel-in-time evaluation of nonlinear recurrences.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, table or helper with the HIP
library in ``newton_evaluation_nonlinear_amd``; the two meet only through the
seeded inputs produced by ``workloads``.

Citations of the form ``[PN §x]`` refer to the web article
"并行牛顿方法：加速非线性序列评估的计算革命" (a survey of parallel Newton methods
for nonlinear sequence evaluation, jsqmd.com news item 789890), section x.

Arithmetic is float64 on the (float32) inputs unless a caller asks for
float32, which is used only to predict failure modes (overflow to non-finite
values) of a single-precision implementation.

Pins (what each function is checked against) live in
``tests/test_oracle_pins.py``; every public function here has at least one.
"""

from .cells import (DiagTanh, TanhRNN, GRU, EulerTanh, make_cell, CELL_DIAG_TANH, CELL_TANH_RNN,
                    CELL_GRU, CELL_EULER_TANH)
from .solver import (
    JACOBI, PICARD, QUASI_NEWTON, NEWTON, BANDED,
    OK, NOT_CONVERGED, NONFINITE,
    sequential, shift, residual_inf, band, jacobian_approx, affine_recurrence,
    newton_step, solve, solve_advancing, SolveResult,
)

__all__ = [
    "DiagTanh", "TanhRNN", "GRU", "EulerTanh", "make_cell",
    "CELL_DIAG_TANH", "CELL_TANH_RNN", "CELL_GRU", "CELL_EULER_TANH",
    "JACOBI", "PICARD", "QUASI_NEWTON", "NEWTON", "BANDED",
    "OK", "NOT_CONVERGED", "NONFINITE",
    "sequential", "shift", "residual_inf", "band", "jacobian_approx",
    "affine_recurrence", "newton_step", "solve", "solve_advancing", "SolveResult",
]
