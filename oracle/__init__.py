"""CPU oracle for the HelixLinear forward pass (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""

from .hxq_oracle import *  # noqa: F401,F403
