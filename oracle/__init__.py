"""CPU oracle for the SeKV mixed-resolution decode path.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
HIP library and never imports it.
"""
from .sekv_oracle import *  # noqa: F401,F403
