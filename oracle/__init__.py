"""fp64 CPU oracle of the CSA / HCA attention path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product path.  It shares
no code with the HIP library in ``long_context_sparse_10_amd``.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against closed forms, brute force, library routines
and the figures the pages print.  The recall of the FP4 indexer on a trained
model (99.7%) cannot be reproduced on synthetic data: that comparison is
"parity unpinned" and is reported, not asserted.
"""
from . import csa, formats  # noqa: F401
