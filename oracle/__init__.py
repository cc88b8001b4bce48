"""CPU oracle for retention-scored KV eviction and renormalised decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
links, imports or calls it, and it shares no code with the HIP library.

``reference`` is the plain, slow definition of every step in float64 (numpy),
written from the pages:

* "Make Each Token Count" (DBTrimKV): Method 2, geometric retention
  r = beta^(t-i); Method 3, one global budget over every layer and head;
  Method 4, paged per-head variable-length KV.
* "Cache What Lasts" (TRIM-KV): Technical summary section 2, the retention
  gate (beta in [0,1]), exponential decay beta^(t-i), evicting the lowest
  current score when the budget M is exceeded.
* "Trust the Mass" (ContourKV): Problem definition (renormalised forced
  weights over the retained set), Method 1 (e_s(A)), Method 3 (dropped-mass
  statistic and allocation).

``brute`` restates selection and attention in pure Python for tiny inputs.

Parity status: every function is pinned by the CPU tests in
``tests/test_oracle_pins.py``.  Three readings stay "parity unpinned",
fixed only by the written specification and not by the pages: the direction
of ties across heads (within a head, the more recent entry first is pinned
by the beta = 1 invariant); the compaction layout and page-table format as
rules (the oracle is pinned against an independent construction of the
same rule); and the allocation's re-offer of units that a cap turns away
(the uncapped largest-remainder rule is pinned by its least-squares
property).
"""
