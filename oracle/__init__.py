"""CPU oracle for the DMS hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  It shares no code with the HIP library.
"""
from .dms_oracle import *  # noqa: F401,F403
from . import dms_oracle  # noqa: F401
from . import dms_train_oracle  # noqa: F401
from . import kvzap_oracle  # noqa: F401
