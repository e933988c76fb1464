"""CPU oracle for the NOSA decode-step hot path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. The HIP library never calls it and shares no code with it.
"""

from .nosa_oracle import *  # noqa: F401,F403
