"""CPU float64 oracle for the KDA state recurrence and its front end — test
infrastructure.

Only tests, the package's smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never imports it and it imports nothing
from the GPU library.  Every function is pinned by the CPU-only tests in
tests/test_oracle_pins.py, tests/test_front_end_pins.py and
tests/test_ring_pins.py against closed
forms, brute force, library routines and the values the pages print.
"""
from .kda_oracle import *  # noqa: F401,F403
from .kda_oracle import __all__ as _recurrence_all
from .front_end import *  # noqa: F401,F403
from .front_end import __all__ as _front_end_all
from .ring import *  # noqa: F401,F403
from .ring import __all__ as _ring_all

__all__ = list(_recurrence_all) + list(_front_end_all) + list(_ring_all)
