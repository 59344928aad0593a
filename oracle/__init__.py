"""Plain, slow CPU oracle for the Mamba-2 SSD chunked scan.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
constants or helpers with the HIP library; the only thing both sides consume
is the seeded input generator (``mamba_ssd_chunked_03_amd.inputs``), which
holds none of the method's arithmetic.

Sources (the pages' own equations were lost in extraction; the formulas used
are the Mamba-2 selective-SSM recurrence in its standard form, written out in
each function, and every function cites the passage it follows):

* gigipick.blogspot.com, "LLM Mamba ...": section 1 (the selective SSM as a
  linear recurrence, h_t needs h_{t-1}), section 2 (the scan element pair and
  the associative combine, Hillis-Steele pseudo-code), section 3 (chunk carry:
  the final state of one chunk seeds the next).
* aitrends.kr/articles/109906, "Helion-based B200 kernel redesign": the
  sequential state-passing loops (forward and backward) turned into an
  associative scan.

Modules
-------
``scan``        the combine operator and three host scans (sequential fold,
                double-buffered Hillis-Steele, Blelloch).
``recurrence``  the literal token-by-token fp64 recurrence, forward and its
                adjoint (backward) with segment checkpoints.  This is the
                oracle the GPU path is checked against.
``chunked``     the four-stage chunked form in fp64 (cumsum, chunk states,
                state passing, chunk output) and its backward.  Used to pin
                ``recurrence`` and to give per-stage intermediates.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, a textbook IIR filter, brute force, finite differences,
an independent autograd, invariants).  None is "parity unpinned".
"""
