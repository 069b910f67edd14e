"""CPU oracle for the RHT + W4A8 / W8A8 quantized linear.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the CPU-baseline
leg of bench.py may import this package.  It shares no code with the HIP
library or its binding, and neither side imports the other.

svg_oracle -- the method step by step (numpy; fp32 where an fp32 operation
              decides an integer code, fp64 for the reference output).
brute      -- pure-Python textbook definitions used to pin svg_oracle on tiny
              inputs.

Parity of every oracle function is pinned by tests in tests/test_oracle.py;
none is marked unpinned.
"""
from . import svg_oracle, brute  # noqa: F401
from .svg_oracle import *  # noqa: F401,F403
