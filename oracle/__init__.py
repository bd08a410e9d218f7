"""Float64 CPU oracle for low-rank-key (Loki-style) sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run this package; the product
path (the HIP library and its Python binding) never does, and shares no code
with it.  It is written to be read against the pages, not to be fast.

Every function is pinned by CPU tests against facts that do not come from the
oracle itself (rotation invariance, full-rank/full-k equivalence with dense
attention, brute-force top-k on tiny inputs, closed forms); see the test file
of oracle pins.
"""

from . import aqua, asym  # noqa: F401
from .calibrate import calibrate, energy_fraction, fix_signs  # noqa: F401
from .loki import (approx_scores, attend, decode, decode_varlen, dense, project,  # noqa: F401
                   rotate_queries, select, topk_indices)
