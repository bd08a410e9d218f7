"""Seeded synthetic inputs for low-rank-key sparse decode attention.

This package is shared by the float64 oracle's tests and by the GPU path's
tests and benchmark.  It holds no step of the method itself (no projection
``K·P``, no scoring, no selection, no softmax): it only draws the cached keys,
values, queries and orthonormal bases that both sides then consume bit for
bit.  Everything is drawn in float64 with NumPy and rounded once to the
storage dtype (fp32 or bf16, round-to-nearest-even by torch's cast).
"""

from .configs import CONFIGS, Config, config  # noqa: F401
from .gen import (make_basis, make_inputs, make_integer_inputs,  # noqa: F401
                  make_query_samples, ordered_scores_fixture, spectrum)
