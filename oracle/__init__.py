"""CPU oracle for the streaming Voxtral decoder-step hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this package.  It shares no code with
the HIP library and never imports it.
"""
from .oracle import *  # noqa: F401,F403
