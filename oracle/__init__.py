"""CPU oracle for the int8-state GDN/KDA decode path.

Test infrastructure only: the test-suite, the smoke check and the benchmark's
CPU-baseline leg use it.  The product path never imports it.
"""
from .lq_oracle import *  # noqa: F401,F403
