"""Plain CPU oracle for the THD context-parallel layout transform.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or runs this
package.  The only callers allowed are the test suite, ``smoke()`` in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py``.

The oracle is slow on purpose: it builds per-token index lists, gathers rows with
``numpy.take`` on raw bytes and derives labels slot by slot.  It shares no code,
table or constant with the HIP library; the only thing both sides receive in
common are the seeded inputs made by ``workloads.py``.

Pins (each function is checked against something other than itself in
``tests/test_oracle_*.py``):

* zigzag / contiguous layouts: the per-rank indices printed on the page
  "Packed Sequence 与上下文并行" (§2.4 Ring single-document example, §3.5 worked
  example, §3.10 contiguous split), plus brute force over every small
  composition against two independent constructions (sort key, closed form);
* route: split-matrix row/column sums, compaction invariance, an emulated
  per-rank pack -> all-to-all -> scatter (as the Relax PR #273 page, §5,
  describes its own test), and run decompositions worked by hand;
* swap: the per-rank token streams printed in §3.6 of the same page, the
  round-trip and cp=1 identities;
* label shift / MTP roll / valid mask: the valid mask and the 13-token count
  printed in §3.4 / §3.8, per-shift closed-form counts, and a per-document
  ``numpy.roll`` on unpadded documents; the single-position form
  (``roll_valid_at``) against the whole-batch one on every small case;
* packing: the boundaries, padding and packed stream printed in §3.2-§3.4 of
  the same page, plus hand-worked corner cases (all-pad rows, PAD inside a
  document, rows ending in EOD, a last document without EOD).

Parity unpinned: the values written at masked positions (the pages only say the
positions are cleared; the oracle writes ``fill``).
"""

from .thd_oracle import (  # noqa: F401
    CONTIGUOUS,
    ZIGZAG,
    OracleInputError,
    check_route_boundaries,
    check_roll_boundaries,
    contiguous_rank_tokens,
    zigzag_rank_tokens,
    zigzag_position,
    layout_tokens,
    build_route,
    canonical_runs,
    swap_rows,
    apply_route,
    roll_labels,
    roll_valid_at,
    pack_batch,
)
