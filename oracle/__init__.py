"""fp64 CPU oracle of the decoder block — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It imports nothing from the product package, and the
product package never imports it.

block.py  -- vectorised fp64 NumPy statement of each step of the block.
brute.py  -- a separate scalar-loop statement for tiny shapes.
"""
from . import block, brute  # noqa: F401
