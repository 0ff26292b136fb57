"""The closed-form run rules the route build relies on, checked against the oracle.

The build cuts each zigzag segment ("Packed Sequence 与上下文并行" §2.4: document
k, rank r owns chunks r and 2cp-1-r) at the contiguous ranks' borders (§2.5:
multiples of T/cp) and decides without looking at the neighbouring segment
whether a piece continues the run before it:

* zigzag-row order (rank-major, then document, then front/back chunk): a
  back chunk continues its front chunk only on rank cp-1, a front chunk
  continues the previous document's back chunk only on rank 0;
* token order (document-major, then chunk): only chunk cp (after chunk
  cp-1, both on rank cp-1) and chunk 0 of a later document (after the
  previous document's chunk 2cp-1, both on rank 0) continue a run;

in both orders never a piece that starts on a destination border, and the
documents (empty slots dropped) lie end to end.  Here the rules are written
out in Python and the runs they produce, in both orders, must equal the
oracle's maximal runs of the per-token route (Relax PR #273 §2.1) exactly,
on random batches and on the corner cases that decide a rule: one-token
chunks, borders on document and chunk starts, a document longer than a
share, many empty slots.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W


def rule_runs(cu, cp, total):
    """Runs (first output row, first input row) in zigzag-row order and in
    token order, from the per-segment rules alone."""
    cu = [int(v) for v in cu]
    docs = [(cu[i], cu[i + 1] - cu[i]) for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]
    n, share = len(docs), total // cp
    c = [length // (2 * cp) for _, length in docs]
    a = [start for start, _ in docs]

    def segment(k, q):
        back = q >= cp
        rank = 2 * cp - 1 - q if back else q
        return a[k] + q * c[k], rank * share + a[k] // cp + (c[k] if back else 0), c[k]

    def pieces(tok, length):
        rem = tok % share
        starts = [tok] if rem + length <= share else [tok, tok - rem + share]
        return rem, starts

    by_src = []  # (zigzag row, token)
    for r in range(cp):
        for k in range(n):
            for h in (0, 1):
                tok, src, length = segment(k, 2 * cp - 1 - r if h else r)
                rem, starts = pieces(tok, length)
                merge = (2 * k + h) > 0 and rem != 0 and (r == cp - 1 if h else r == 0)
                for p, ptok in enumerate(starts):
                    if p >= merge:
                        by_src.append((src + ptok - tok, ptok))
    by_tok = []  # (token, zigzag row)
    for k in range(n):
        for q in range(2 * cp):
            tok, src, length = segment(k, q)
            rem, starts = pieces(tok, length)
            merge = rem != 0 and (q == cp or (q == 0 and k > 0))
            for p, ptok in enumerate(starts):
                if p >= merge:
                    by_tok.append((ptok, src + ptok - tok))
    return by_src, by_tok


def with_lengths(runs, total):
    """(first out, first in) pairs in output order -> (out, in, length)."""
    outs = [o for o, _ in runs] + [total]
    return np.array([(o, i, outs[j + 1] - o) for j, (o, i) in enumerate(runs)], dtype=np.int64).reshape(-1, 3)


def check(cu, cp, total):
    by_src, by_tok = rule_runs(cu, cp, total)
    want = O.canonical_runs(O.build_route(cu, cp, total))       # (zigzag row, token, length), by zigzag row
    got_src = with_lengths(by_src, total)
    assert np.array_equal(got_src, want), (list(cu), cp)
    want_tok = want[np.argsort(want[:, 1], kind="stable")][:, [1, 0, 2]]   # the same runs by token
    got_tok = with_lengths(by_tok, total)
    assert np.array_equal(got_tok, want_tok), (list(cu), cp)


@pytest.mark.parametrize("cp", [2, 3, 4, 5, 8, 16])
def test_rules_on_random_batches(cp):
    rng = np.random.default_rng([W.BASE_SEED, 31, cp])
    for _ in range(60):
        n = int(rng.integers(1, 14))
        lengths = (rng.integers(0, 7, n) * 2 * cp).tolist()       # zeros are empty slots
        if sum(lengths) == 0:
            lengths[0] = 2 * cp
        cu = np.concatenate([[0], np.cumsum(lengths)])
        check(cu, cp, int(cu[-1]))


@pytest.mark.parametrize("cu,cp", [
    ([0, 4, 8, 16], 2),                  # the page's worked example (§3)
    ([0, 8, 20, 24], 2),                 # a run that crosses from one document into the next
    ([0, 8], 2),                         # one document (§2.4's single-document example)
    ([0, 4, 4, 8, 8, 8, 12], 2),         # one-token chunks, empty slots between documents
    ([0, 16, 32], 4),                    # each document exactly one share: borders on document starts
    ([0, 64], 4),                        # one document spanning every share
    ([0, 8, 72], 4),                     # a long document after a short one: borders inside chunks
    ([0, 24, 24, 48], 3),                # cp 3, borders on chunk starts
    ([0, 32, 96, 128], 16),              # one-token chunks with cp 16
])
def test_rules_on_corner_cases(cu, cp):
    check(np.array(cu), cp, cu[-1])


def test_rules_on_the_configured_workloads():
    for name in ("tiny", "gdn128k", "sft", "sft512", "full"):
        w = W.make(name)
        check(w.cu_padded, w.cp, w.total)
