"""CPU oracle — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 (numpy) statement of what the hot path
computes. It exists to check the HIP library and nothing else: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It shares no code with the library (no kernels, headers, helpers or
constant tables) and never imports it; the only module both sides use is the
seeded input generator ``synth``, which holds none of the method's arithmetic.

Modules (each function cites the passage of the source pages it follows):
  * ``w4``        — int4 group-32 dequantisation, the m-row GEMV, the routed
                    (mixture-of-experts) GEMV and its distinct-expert byte count;
  * ``attention`` — extend-prefill attention (m new rows against a cached
                    prefix plus themselves), vectorised and brute-force forms,
                    and several questions about one cached state;
  * ``slots``     — the resident KV-slot store and the slot-selection rule;
  * ``fit``       — the fixed + marginal-per-row cost fit of verify time;
  * ``verify``    — greedy acceptance of a verify step, the KV rollback it
                    implies, the rolling-acceptance gate and the break-even
                    acceptance of the cost model;
  * ``ngram``     — prompt-lookup drafting (the tokens that followed the
                    latest earlier occurrence of the history's suffix).

Every function here is pinned by ``tests/test_oracle_*.py`` to closed forms,
invariants, brute force or independent library routines; none is left
"parity unpinned".
"""
