"""CPU oracle for the routed-MoE expert path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and nothing here
imports the product path: the two share no code.  Inputs come from
``moe_synth`` (seeded generators with none of the method's arithmetic).

Every function is a plain, slow, fp64 restatement of what the four source pages
define; see ``oracle.moe_oracle`` for the per-function citations.  Parity pins
for every function live in ``tests/test_oracle_pins.py``; no function here is
"parity unpinned".
"""
from .moe_oracle import *  # noqa: F401,F403
