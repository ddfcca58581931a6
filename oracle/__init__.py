"""CPU oracle for the codebook-LUT MoE path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and it
shares no code, table or helper with that path.

It is a plain, slow, obviously-correct restatement of what the method computes,
in fp64 unless a step fixes another precision.  See ``reference.py`` for every
function and the passage of the CodeQuant / CodeQuant2 pages it follows.

Pins (what ties each function to something other than itself) live in
``tests/test_oracle_*.py``; every function here is pinned.  The only quantity the
pages would let us check end to end - model accuracy or speed - needs trained
weights and datasets that are not available, so the layer as a whole is pinned
only by the mathematics (closed forms, brute force, invariants), not by a number
printed on the pages.
"""
from .reference import *  # noqa: F401,F403
from .reference import __all__  # noqa: F401
