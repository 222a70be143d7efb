"""fp64 CPU oracle for the multi-LoRA delta path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""
from .lora_oracle import *  # noqa: F401,F403
from .lora_oracle import PINS  # noqa: F401
