"""CPU oracle for the SVDQuant W4A4 linear layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the C-ABI library and its
Python binding) never calls it and shares no code with it.
"""

from .svdq_oracle import *  # noqa: F401,F403
from .mxfp4_oracle import *  # noqa: F401,F403
from .w4a16_oracle import *  # noqa: F401,F403
