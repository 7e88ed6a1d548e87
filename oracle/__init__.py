"""CPU oracle of the Kamera reuse operator (test infrastructure only).

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; never by the product package.
"""

from .kamera_oracle import *  # noqa: F401,F403
