"""CPU oracle for the Mamba-3 MIMO backward first stage.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import, call, link or execute anything in
this package. The product path (``mamba_mimo_chunked_amd``) never does, and the
two share no code.

* ``o1``  -- contract oracle (C, token-by-token loops, the pages' bf16/fp32
  rounding points; ``exact=True`` turns every rounding off and carries float64).
  This is the parity reference for the HIP path.
* ``o2_sequential`` -- exact unchunked recurrence (numpy float64).
* ``o3_bruteforce`` -- exact quadratic form over all token pairs (tiny inputs).
"""
