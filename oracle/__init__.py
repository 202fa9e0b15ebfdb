"""Plain, slow CPU oracle for the large-beam Gated DeltaNet decode step (numpy, float64).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of the benchmark are
the only code that may import it.  It shares no code with the HIP library and the library never calls
it: when the HIP extension is missing, the product path fails instead of falling back to this.

Every function is pinned by tests under ``tests/`` marked "not gpu": agreement of the two independent
forms (dense FullState vs record replay) on tiny inputs, exact rational brute force of the gated delta
rule, closed forms (beta = 0; alpha = beta = 1 with orthonormal keys; S_ctx = 0; linearity), beam
relabelling and duplication invariants, and a hand-written ancestry table.
"""

from .gdn_beam import *  # noqa: F401,F403
from .gdn_beam import __all__  # noqa: F401
