"""CPU oracle for the W8A8 INT8 linear layer -- TEST INFRASTRUCTURE ONLY.

This package is the checker, not the product. Only the test suite, the
``smoke()`` entry of ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it. The HIP library never calls it and shares no code
with it.

Everything lives in :mod:`oracle.w8a8_oracle`; see its header for what each
function follows and how it is pinned.
"""

from .w8a8_oracle import *  # noqa: F401,F403
from .w8a8_oracle import __all__  # noqa: F401
