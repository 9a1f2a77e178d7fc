"""CPU oracle of the QuantSparse attention hot path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  See ``qsa_oracle`` for what it computes.
"""
from .qsa_oracle import *  # noqa: F401,F403
from .qsa_oracle import __all__  # noqa: F401
