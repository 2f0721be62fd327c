"""CPU oracle of the RTPurbo sparse-attention decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.
"""
from .rtp_oracle import *  # noqa: F401,F403
from .cluster_index import *  # noqa: F401,F403,E402
