"""Brute-force and invariant pins of the CPU oracle (CPU only).

The oracle builds the zigzag layout by appending each rank's chunk ranges.  Two
independent constructions written here must agree with it on every small
input:

* sort key: give every token the key (owning rank, slot, back half?, offset)
  and sort;
* closed form: the row of token g in slot s, chunk q = (g - cu[s]) // c is
  rank(q) * T/cp + cu[s]/cp + (q >= cp) * c + (g - cu[s] - q*c), with
  rank(q) = q for q < cp and 2*cp-1-q otherwise.
"""

import itertools

import numpy as np
import pytest

import oracle as O
import workloads as W


def compositions(total_units, max_parts=None):
    """All ordered ways of writing total_units as a sum of positive parts."""
    if total_units == 0:
        yield []
        return
    for first in range(1, total_units + 1):
        for rest in compositions(total_units - first):
            out = [first] + rest
            if max_parts is None or len(out) <= max_parts:
                yield out


def with_empty_slots(lengths, n_empty):
    """Every placement of n_empty zero-length slots among the documents."""
    n = len(lengths)
    for pos in itertools.combinations_with_replacement(range(n + 1), n_empty):
        out = list(lengths)
        for p in reversed(pos):
            out.insert(p, 0)
        yield out


def sort_key_order(cu, cp):
    keys = []
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        if L == 0:
            continue
        c = L // (2 * cp)
        for g in range(cu[s], cu[s + 1]):
            q = (g - cu[s]) // c
            rank = q if q < cp else 2 * cp - 1 - q
            keys.append((rank, s, q >= cp, g - cu[s], g))
    keys.sort()
    return [k[-1] for k in keys]


def closed_form_rows(cu, cp, total):
    rows = [None] * total
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        if L == 0:
            continue
        c = L // (2 * cp)
        for g in range(cu[s], cu[s + 1]):
            q = (g - cu[s]) // c
            rank = q if q < cp else 2 * cp - 1 - q
            rows[g] = rank * (total // cp) + cu[s] // cp + (c if q >= cp else 0) + (g - cu[s] - q * c)
    return rows


def small_cases():
    cases = []
    for cp, max_total in ((1, 16), (2, 24), (3, 24), (4, 24)):
        unit = 2 * cp
        for units in range(0, max_total // unit + 1):
            for comp in compositions(units):
                lens = [unit * u for u in comp]
                n_empty_opts = (0, 1) if cp == 1 else (0, 1, 2)
                for ne in n_empty_opts:
                    if ne and len(lens) > 4:
                        continue
                    for lens_e in with_empty_slots(lens, ne):
                        if not lens_e:
                            continue
                        cases.append((cp, W.cumulative(lens_e).tolist()))
    return cases


CASES = small_cases()


def test_case_count_is_substantial():
    assert len(CASES) > 1000


@pytest.mark.parametrize("cp", [1, 2, 3, 4])
def test_zigzag_matches_sort_key_and_closed_form(cp):
    n = 0
    for cpc, cu in CASES:
        if cpc != cp:
            continue
        total = cu[-1]
        z = O.layout_tokens(cu, cp, total, O.ZIGZAG)
        assert z.tolist() == sort_key_order(cu, cp), cu
        pos = np.empty(total, np.int64)
        pos[z] = np.arange(total)
        assert pos.tolist() == closed_form_rows(cu, cp, total), cu
        n += 1
    assert n > 10


@pytest.mark.parametrize("cp", [1, 2, 3, 4])
def test_single_token_form_matches_the_lists(cp):
    # zigzag_position (used to check huge batches token by token) against the
    # per-rank lists, on every small case.
    for cpc, cu in CASES:
        if cpc != cp:
            continue
        total = cu[-1]
        z = O.layout_tokens(cu, cp, total, O.ZIGZAG)
        for row, g in enumerate(z.tolist()):
            assert O.zigzag_position(cu, cp, total, g) == row, (cu, g)


@pytest.mark.parametrize("cp", [2, 3, 4])
def test_route_invariants(cp):
    rng = np.random.default_rng(7)
    for cpc, cu in CASES:
        if cpc != cp:
            continue
        total = cu[-1]
        route = O.build_route(cu, cp, total)
        share = total // cp
        split = route["split"]
        # each rank sends and receives exactly its share
        assert (split.sum(axis=1) == share).all() and (split.sum(axis=0) == share).all()
        # what rank s lists as sent to d equals what d lists as received from s
        for s in range(cp):
            assert route["input_split_sizes"][s].tolist() == [split[s, d] for d in range(cp)]
        for d in range(cp):
            assert route["output_split_sizes"][d].tolist() == [split[s, d] for s in range(cp)]
        # permutation + round trip on random bytes
        x = rng.integers(0, 256, size=(total, 3), dtype=np.uint8)
        y = O.swap_rows(x, cu, cp, total, "z2c")
        assert sorted(map(bytes, y)) == sorted(map(bytes, x))
        assert np.array_equal(O.swap_rows(y, cu, cp, total, "c2z"), x)
        # runs expand back to the per-token map and are maximal
        runs = O.canonical_runs(route)
        if total:
            src = np.concatenate([np.arange(a, a + n) for a, _, n in runs])
            dst = np.concatenate([np.arange(b, b + n) for _, b, n in runs])
            assert src.tolist() == list(range(total))
            assert np.array_equal(route["dst_row"][route["zigzag"]][src], dst)
            for (a0, b0, n0), (a1, b1, _) in zip(runs[:-1], runs[1:]):
                joinable = (b1 == b0 + n0 and a1 == a0 + n0
                            and a1 % share != 0 and b1 % share != 0)
                assert not joinable
            # bound on the run count: 2*cp*docs + cp - 1
            docs = sum(1 for i in range(len(cu) - 1) if cu[i + 1] > cu[i])
            assert len(runs) <= 2 * cp * docs + cp - 1


@pytest.mark.parametrize("cp", [2, 4])
def test_compaction_invariance(cp):
    # Empty slots (repeated boundaries) never change the route.
    for cpc, cu in CASES:
        if cpc != cp:
            continue
        total = cu[-1]
        compact = [cu[0]] + [cu[i + 1] for i in range(len(cu) - 1) if cu[i + 1] > cu[i]]
        a = O.build_route(cu, cp, total)
        b = O.build_route(compact, cp, total)
        assert np.array_equal(a["zigzag"], b["zigzag"])
        assert np.array_equal(a["split"], b["split"])


@pytest.mark.parametrize("seed", range(6))
def test_emulated_all_to_all_matches_global_swap(seed):
    # Relax PR #273 §2.1 / §5: pack -> all-to-all -> scatter on every rank,
    # simulated locally, equals the one global permutation.
    cp = [2, 3, 4, 8, 2, 4][seed]
    w = W.random_packed(seed, cp, n_docs=5 + seed, max_chunk=6, n_empty=seed % 3)
    cu, total = w.cu_padded.tolist(), w.total
    route = O.build_route(cu, cp, total)
    share = total // cp
    x = w.rows_host()
    zig = x                                        # emulated zigzag buffer (any content)
    recv = {d: [] for d in range(cp)}
    for s in range(cp):
        local = zig[s * share:(s + 1) * share]
        send = local[route["send_rows"][s]]
        pieces = np.split(send, np.cumsum(route["input_split_sizes"][s])[:-1])
        for d in range(cp):
            recv[d].append(pieces[d])
    out = np.empty_like(zig)
    for d in range(cp):
        buf = np.concatenate(recv[d])
        assert buf.shape[0] == route["output_split_sizes"][d].sum() == share
        local_out = np.empty_like(buf)
        local_out[route["recv_rows"][d]] = buf
        out[d * share:(d + 1) * share] = local_out
    assert np.array_equal(out, O.swap_rows(zig, cu, cp, total, "z2c"))


@pytest.mark.parametrize("seed", range(4))
def test_route_applied_piece_by_piece_equals_the_whole_swap(seed):
    # Applying a built route to slices of output rows and stacking them gives
    # the one-shot swap (the form used to check batches too large to gather
    # at once); the route is built once and applied in both directions.
    cp = [2, 3, 4, 8][seed]
    w = W.random_packed(40 + seed, cp, n_docs=6 + seed, max_chunk=7, n_empty=seed % 2)
    cu, total = w.cu_padded.tolist(), w.total
    route = O.build_route(cu, cp, total)
    x = w.rows_host()
    for direction in ("z2c", "c2z"):
        whole = O.swap_rows(x, cu, cp, total, direction)
        assert np.array_equal(O.apply_route(x, route, direction), whole)
        step = max(1, total // 5 + 1)
        pieces = [O.apply_route(x, route, direction, slice(a, min(a + step, total))) for a in range(0, total, step)]
        assert np.array_equal(np.concatenate(pieces), whole)
    # an identity route hands the input back
    one = O.build_route(cu, 1, total)
    assert O.apply_route(x, one, "z2c") is x


def test_roll_matches_per_document_numpy_roll():
    # Unpadded documents: shift j inside a document is np.roll(doc, -j) with the
    # last j positions cleared.
    rng = np.random.default_rng(11)
    lens = [5, 1, 9, 3, 0, 12]
    cu = W.cumulative(lens)
    total = int(cu[-1])
    ids = rng.integers(0, 32000, size=total, dtype=np.int64)
    shifted, mask = O.roll_labels(ids, cu, None, total, 4, fill=-7)
    for s, L in enumerate(lens):
        a = int(cu[s])
        doc = ids[a:a + L]
        for j in range(1, 5):
            want = np.roll(doc, -j).copy()
            want[max(0, L - j):] = -7
            assert shifted[j - 1, a:a + L].tolist() == want.tolist()
            assert mask[j, a:a + L].tolist() == [1] * max(0, L - j) + [0] * min(L, j)
    assert mask[0].all()


@pytest.mark.parametrize("seed", range(5))
def test_roll_counts_and_no_crossing(seed):
    w = W.random_packed(seed, 2, n_docs=7, max_chunk=5, n_empty=2, pad_max=3)
    total = w.total
    ids = np.arange(total, dtype=np.int64) + 100     # ids reveal their position
    shifted, mask = O.roll_labels(ids, w.cu_padded, w.cu_real, total, 4, fill=-1)
    real = np.diff(w.cu_real)
    for j in range(0, 5):
        assert int(mask[j].sum()) == int(np.maximum(real - j, 0).sum())
    # a target at position t is token t + j of the same document, never a pad
    slot_of = np.searchsorted(w.cu_padded, np.arange(total), side="right") - 1
    for j in range(1, 5):
        for t in np.flatnonzero(mask[j]):
            src = int(shifted[j - 1, t]) - 100
            assert src == t + j
            assert slot_of[src] == slot_of[t]
            assert src < w.cu_padded[slot_of[t]] + real[slot_of[t]]
        assert (shifted[j - 1][mask[j] == 0] == -1).all()


def test_workload_recipes():
    for name in W.NAMES + ("sft512",):
        w = W.make(name)
        L = np.diff(w.cu_padded.astype(np.int64))
        R = np.diff(w.cu_real.astype(np.int64))
        assert w.cu_padded[0] == 0 and (L >= 0).all()
        assert (L % (2 * w.cp) == 0).all()
        assert (R <= L).all() and (R >= 0).all()
    assert W.make("gdn128k").total == 131072 and W.make("sft").total == 131072
    assert W.make("long1m").total == 1048576 and W.make("full").total == 262144
    sft = W.make("sft")
    assert int((np.diff(sft.cu_padded) == 0).sum()) == 8 and sft.cu_padded[-1] == sft.cu_padded[-2]
    assert int((np.diff(W.make("sft512").cu_padded) > 0).sum()) == 512
    assert (np.diff(W.make("full").cu_padded) % 512 == 0).all()
    assert W.make("long1m").n_slots == 6
    # seeded: the same recipe gives the same batch
    assert np.array_equal(W.make("full").cu_padded, W.make("full").cu_padded)


def test_single_position_roll_form_matches_the_batch_form():
    # roll_valid_at (used to check huge batches position by position) against
    # roll_labels on random small batches with pads, empty slots and every shift.
    rng = np.random.default_rng(11)
    for _ in range(60):
        n = int(rng.integers(1, 7))
        padded = [int(rng.integers(0, 6)) * 4 for _ in range(n)]
        real = [int(rng.integers(0, p + 1)) for p in padded]
        cu_p = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
        cu_r = np.concatenate([[0], np.cumsum(real)]).astype(np.int64)
        total = int(cu_p[-1])
        if total == 0:
            continue
        ids = rng.integers(0, 1000, size=total)
        shifted, mask = O.roll_labels(ids, cu_p, cu_r, total, 4, -7)
        for t in range(total):
            for j in range(5):
                ok = O.roll_valid_at(cu_p, cu_r, t, j)
                assert mask[j, t] == ok, (cu_p, cu_r, t, j)
                if j:
                    assert shifted[j - 1, t] == (ids[t + j] if ok else -7)
    with pytest.raises(O.OracleInputError):
        O.roll_valid_at([0, 4], [0, 4], 4, 0)
