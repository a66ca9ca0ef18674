"""CPU oracle of the row-wise RMSNorm family: plain FP64 numpy, written from the pages.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything here.  The
GPU library (``dit_normalization_amd``) never imports it and shares no code with it: the two
meet only through the seeded inputs of ``workloads``.

Parity status: every public function is pinned by ``tests/test_oracle_*.py`` to something
other than itself (format definitions and brute-force searches, torch CPU library routines,
closed forms, invariants, finite differences, exactly rounded sums).
"""
from . import formats, rmsnorm  # noqa: F401
