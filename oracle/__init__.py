"""CPU oracle for the SharQ linear-layer hot path -- TEST INFRASTRUCTURE ONLY.

Plain numpy implementation of what the GPU library computes, written from the
pages about SharQ (see ``oracle.sharq`` and ``oracle.formats`` for the passages
each step follows).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
cpu_baseline leg of ``bench.py`` may import it.  It shares no code with the GPU
path; the product path must never route through it.

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/`` (hand
fixtures under ``tests/golden/``, closed forms, brute force, the pages'
identities).  Parity unpinned: the relative Frobenius errors of SharQ and of
plain FP4 are reported, not checked against printed values (the pages print
none for synthetic inputs); only their ordering is tested.
"""
from . import formats, sharq  # noqa: F401
