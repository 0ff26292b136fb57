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

For batches of many documents the build places runs without a scan: the
runs before segment j of an order number j, less the rule merges before it,
plus every destination border before it that falls inside a segment or on
the start of one the rules would have merged; and the split matrix follows
per destination share from the two documents at its ends plus 2 c for every
document between.  Those formulas, written out here, must match the rules
segment by segment and the oracle's run count and split matrix.
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


def closed_form(cu, cp, total):
    """The slot formulas of the closed-form build: for segment j of each
    order, the number of runs the segments before it produce, and the split
    matrix, from the documents and the cp - 1 destination borders alone."""
    cu = [int(v) for v in cu]
    docs = [(cu[i], cu[i + 1] - cu[i]) for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]
    n, share, two_cp = len(docs), total // cp, 2 * cp
    a = [start for start, _ in docs]
    c = [length // two_cp for _, length in docs]

    def doc_at(t):
        return max(k for k in range(n) if a[k] <= t)

    # the document of every border b * share, b = 0 .. cp - 1, as the build
    # finds it: from each document, the borders inside [a_k, a_k + 2 cp c_k)
    # (the documents lie end to end, so each border is in exactly one)
    border_doc = {}
    for k in range(n):
        b = -(-a[k] // share)
        while b < cp and b * share < a[k] + two_cp * c[k]:
            assert b not in border_doc
            border_doc[b] = k
            b += 1
    assert sorted(border_doc) == list(range(cp))
    assert all(border_doc[b] == doc_at(b * share) for b in range(cp))

    # each border that adds a run: inside a segment (a second piece), or on the
    # start of a segment the rules would have merged
    add_s, add_t = [], []
    for b in range(1, cp):
        t = b * share
        k = border_doc[b]
        q = (t - a[k]) // c[k]
        inside = t - a[k] != q * c[k]
        back = q >= cp
        r, rem = (two_cp - 1 - q if back else q), 2 * k + (1 if back else 0)
        if inside or (rem > 0 and (r == cp - 1 if back else r == 0)):
            add_s.append(r * 2 * n + rem)
        if inside or q == cp or (q == 0 and k > 0):
            add_t.append(k * two_cp + q)

    def merges_zigzag(j):
        r, rem = divmod(j, 2 * n)
        if r >= cp:
            return 2 * n - 1
        if r == 0:
            return (rem - 1) // 2 if rem >= 1 else 0
        return n - 1 if r < cp - 1 else n - 1 + rem // 2

    def merges_token(j):
        k, q = divmod(j, two_cp)
        return (2 * k - 1 if k >= 1 else 0) + (1 if k >= 1 and q > 0 else 0) + (1 if q > cp else 0)

    def runs_before_zigzag(j):
        return j - merges_zigzag(j) + sum(1 for e in add_s if e < j)

    def runs_before_token(j):
        return j - merges_token(j) + sum(1 for e in add_t if e < j)

    def rank_tokens_in(k, s, lo, hi):
        return sum(max(0, min(x + c[k], hi) - max(x, lo)) for x in (a[k] + s * c[k], a[k] + (two_cp - 1 - s) * c[k]))

    split = np.zeros((cp, cp), dtype=np.int64)
    for d in range(cp):
        lo, hi = d * share, (d + 1) * share
        # the document holding token hi - 1: that of border d + 1, or the one
        # before it when the border starts a document
        k0 = border_doc[d]
        if d + 1 < cp:
            k_hi = border_doc[d + 1]
            k1 = k_hi - 1 if a[k_hi] == hi else k_hi
        else:
            k1 = n - 1
        assert (k0, k1) == (doc_at(lo), doc_at(hi - 1))
        for s_ in range(cp):
            v = rank_tokens_in(k0, s_, lo, hi)
            if k1 > k0:   # documents between hold 2 c of every rank; a_k / (2 cp) sums c before k
                v += rank_tokens_in(k1, s_, lo, hi) + 2 * (a[k1] - a[k0 + 1]) // two_cp
            split[s_, d] = v
    return n, runs_before_zigzag, runs_before_token, split


def add_s_list(cu, cp, total):
    """Zigzag-order segment index r * 2n + rem of every border that adds a run."""
    cu = [int(v) for v in cu]
    docs = [(cu[i], cu[i + 1] - cu[i]) for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]
    n, share, two_cp = len(docs), total // cp, 2 * cp
    out = []
    for b in range(1, cp):
        t = b * share
        k = max(i for i in range(n) if docs[i][0] <= t)
        a, c = docs[k][0], docs[k][1] // two_cp
        q = (t - a) // c
        back = q >= cp
        r, rem = (two_cp - 1 - q if back else q), 2 * k + (1 if back else 0)
        if t - a != q * c or (rem > 0 and (r == cp - 1 if back else r == 0)):
            out.append(r * 2 * n + rem)
    return out


def check_closed_form(cu, cp, total):
    n, before_s, before_t, split = closed_form(cu, cp, total)
    by_src, by_tok = rule_runs(cu, cp, total)
    route = O.build_route([int(v) for v in cu], cp, total)
    assert np.array_equal(split, route["split"]), (list(cu), cp)
    runs = O.canonical_runs(route)
    # the slot of a segment's first new run is the number of runs before it:
    # walk the rules segment by segment and compare at every segment
    cu_l = [int(v) for v in cu]
    docs = [(cu_l[i], cu_l[i + 1] - cu_l[i]) for i in range(len(cu_l) - 1) if cu_l[i + 1] > cu_l[i]]
    share, two_cp = total // cp, 2 * cp
    a = [d[0] for d in docs]
    c = [d[1] // two_cp for d in docs]
    # the build keys zigzag-order borders by r * (2 n_slots) + rem before it
    # knows n: the same count before every segment as keys r * 2n + rem
    stride = 2 * (len(cu_l) - 1)
    add_s_keys = [(e // (2 * n)) * stride + e % (2 * n) for e in add_s_list(cu_l, cp, total)]
    for j in range(two_cp * n + 1):
        r, rem = divmod(j, 2 * n)
        key = r * stride + rem if j < two_cp * n else float("inf")
        assert sum(1 for e in add_s_keys if e < key) == sum(1 for e in add_s_list(cu_l, cp, total) if e < j)
    count = 0
    for j in range(two_cp * n):
        assert before_s(j) == count, (list(cu), cp, "zigzag", j)
        r, rem = divmod(j, 2 * n)
        k, h = rem >> 1, rem & 1
        tok = a[k] + (two_cp - 1 - r if h else r) * c[k]
        cut = tok % share
        count += (2 if cut + c[k] > share else 1) - (1 if rem > 0 and cut != 0 and (r == cp - 1 if h else r == 0) else 0)
    assert before_s(two_cp * n) == count == len(runs) == len(by_src)
    count = 0
    for j in range(two_cp * n):
        assert before_t(j) == count, (list(cu), cp, "token", j)
        k, q = divmod(j, two_cp)
        tok = a[k] + q * c[k]
        cut = tok % share
        count += (2 if cut + c[k] > share else 1) - (1 if cut != 0 and (q == cp or (q == 0 and k > 0)) else 0)
    assert before_t(two_cp * n) == count == len(runs) == len(by_tok)


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


@pytest.mark.parametrize("cp", [2, 3, 4, 5, 8, 16, 32])
def test_closed_form_slots_and_split_on_random_batches(cp):
    # The formulas route_runs_kernel places runs and fills the split matrix
    # with: runs before every segment of each order equal the running count of
    # the rules, the totals equal the oracle's run count, and the split
    # matrix equals the oracle's.
    rng = np.random.default_rng([W.BASE_SEED, 32, cp])
    for _ in range(40):
        n = int(rng.integers(1, 14))
        lengths = (rng.integers(0, 7, n) * 2 * cp).tolist()
        if sum(lengths) == 0:
            lengths[0] = 2 * cp
        cu = np.concatenate([[0], np.cumsum(lengths)])
        check_closed_form(cu, cp, int(cu[-1]))


@pytest.mark.parametrize("cu,cp", [([0, 4, 8, 16], 2), ([0, 16, 32], 4), ([0, 64], 4), ([0, 8, 72], 4),
                                   ([0, 24, 24, 48], 3), ([0, 32, 96, 128], 16)])
def test_closed_form_on_corner_cases(cu, cp):
    check_closed_form(np.array(cu), cp, cu[-1])


def test_closed_form_on_the_many_document_workload():
    w = W.make("sft512")
    check_closed_form(w.cu_padded, w.cp, w.total)
