"""CPU oracle of the SPD draft-and-verify cycle.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product package.  See oracle/spd.py
for the pages it follows and the pins that check it.
"""
from . import spd  # noqa: F401
from . import cycle  # noqa: F401
