"""Query-dependent dynamic sparse attention on AMD MI355X (gfx950).

The computation lives in libsa.so (HIP kernels behind the C ABI declared in
include/sa.h); ``ops`` is the thin torch binding with the same entry-point
names.  There is no CPU fallback: calls raise if the library is not built.
"""

from . import _lib  # noqa: F401
from ._lib import SAError  # noqa: F401

__version__ = "0.1.0"


def load_library():
    """Load libsa.so (raises ImportError with build instructions if missing)."""
    return _lib.load()
