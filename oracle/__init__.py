"""CPU oracle for the verify-pass weight stream (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls anything under ``oracle/``.
"""
from .verify_oracle import *  # noqa: F401,F403
from .sampling_oracle import *  # noqa: F401,F403
from .gdn_oracle import *  # noqa: F401,F403
