"""Plain, slow CPU oracle for the large-beam Gated DeltaNet decode step (numpy, float64) and for the beam
selection that feeds it its parents.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of the benchmark are
the only code that may import it.  It shares no code with the HIP library and the library never calls
it: when the HIP extension is missing, the product path fails instead of falling back to this.

Every function is pinned by tests under ``tests/`` marked "not gpu": agreement of the two independent
forms (dense FullState vs record replay) on tiny inputs, exact rational brute force of the gated delta
rule, closed forms (beta = 0; alpha = beta = 1 with orthonormal keys; S_ctx = 0; linearity), beam
relabelling and duplication invariants, a hand-written ancestry table; for the beam selection, a
pure-Python brute force, closed forms (one parent; all scores equal; separated parents) and the
top-set invariants.
"""

from .gdn_beam import *  # noqa: F401,F403
from .gdn_beam import __all__ as _gdn_all
from .beam_selection import *  # noqa: F401,F403
from .beam_selection import __all__ as _sel_all

__all__ = list(_gdn_all) + list(_sel_all)
