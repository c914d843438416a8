"""CPU oracle for the decode-time KV-cache compression event.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, header,
table or constant with the HIP library; the only thing both sides consume is
the seeded input generator module, which holds none of the method's arithmetic.

``oracle.ams``   plain NumPy oracle (fp64 window score, exact integer contract
                 for mass / segmentation / quota / select / gather).
``oracle.loops`` pure-Python loop re-statement for tiny shapes, used only to
                 cross-check ``oracle.ams``.
``oracle.refresh`` the RefreshKV decode-loop pieces around the event (query
                 comparison trigger, partial-cache append/evict, full-cache sync).
"""
from . import ams, loops, refresh  # noqa: F401
