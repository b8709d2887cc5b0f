"""Plain CPU oracle for the fused microscaling (MX) mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library in ``block_scaled_precision_amd/``.

Everything here is numpy in float64, written to be read against the pages
rather than to be fast:

* ``oracle.mx``      -- OCP MX element codecs (E2M1, E3M2, E4M3, E8M0), the
                        32-element block quantizer and the canonical byte
                        packing of codes.
* ``oracle.routing`` -- softmax/top-k routing and the permutation of
                        assignments by expert.
* ``oracle.moe``     -- the layer forward: activation quantization, FC1,
                        SiLU(gate)*up with its rounding/requantization point,
                        FC2, routing-weighted combine and the shared expert.

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: hand-listed decode values, torch's own float8 codecs, brute-force
nearest-value search over every bf16 bit pattern, exact rational arithmetic
on tiny GEMMs, closed forms and invariants.  Every function is pinned; none is
"parity unpinned".
"""
