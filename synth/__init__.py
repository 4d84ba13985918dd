"""Seeded synthetic inputs shared by the GPU path tests, the bench and the oracle.

This package draws inputs only: random normal queries/keys/values, projector
weights, planted needles and heavy hitters, sequence lengths and page tables.
It holds none of the sparse-attention arithmetic (no scores, no selection, no
attention) and imports neither the oracle nor the HIP library.
"""

from .gen import *  # noqa: F401,F403
from .gen import __all__  # noqa: F401
