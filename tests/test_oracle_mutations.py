"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a patched copy of an oracle function -- a
wrong chunk index, swapped chunk order, a dropped term, exchanged directions,
an off-by-one at a document end -- and checks that at least one pin from
test_oracle_pins / test_oracle_bruteforce fails on it.  The real oracle is
restored after every case.
"""

import contextlib

import numpy as np
import pytest

import oracle
import oracle.thd_oracle as T
import test_oracle_bruteforce as BF
import test_oracle_pins as P
from conftest import read_golden


def _zig_back_off_by_one(cu, cp, rank):
    b = [int(v) for v in np.asarray(cu).reshape(-1)]
    out = []
    for s in range(len(b) - 1):
        chunk = (b[s + 1] - b[s]) // (2 * cp)
        for c in (rank, 2 * cp - rank - 2 if 2 * cp - rank - 2 >= 0 else 0):
            out.extend(range(b[s] + c * chunk, b[s] + (c + 1) * chunk))
    return np.asarray(out, dtype=np.int64)


def _zig_back_first(cu, cp, rank):
    b = [int(v) for v in np.asarray(cu).reshape(-1)]
    out = []
    for s in range(len(b) - 1):
        chunk = (b[s + 1] - b[s]) // (2 * cp)
        for c in (2 * cp - 1 - rank, rank):
            out.extend(range(b[s] + c * chunk, b[s] + (c + 1) * chunk))
    return np.asarray(out, dtype=np.int64)


def _zig_chunk_by_cp(cu, cp, rank):          # chunk L/cp instead of L/(2cp), truncated to fit
    b = [int(v) for v in np.asarray(cu).reshape(-1)]
    out = []
    for s in range(len(b) - 1):
        chunk = (b[s + 1] - b[s]) // (2 * cp)
        first = b[s] + rank * 2 * chunk
        out.extend(range(first, first + 2 * chunk))
    return np.asarray(out, dtype=np.int64)


def _contig_reversed(total, cp, rank):
    share = total // cp
    r = cp - 1 - rank
    return np.arange(r * share, (r + 1) * share, dtype=np.int64)


_real_swap = T.swap_rows


def _swap_directions_exchanged(x, cu, cp, total, direction):
    other = {"z2c": "c2z", "c2z": "z2c"}.get(direction, direction)
    return _real_swap(x, cu, cp, total, other)


_real_apply = T.apply_route


def _apply_gathers_by_the_inverse(x, route, direction, out_rows=None):
    # gathers with the row list of the other direction (the inverse permutation)
    other = {"z2c": "c2z", "c2z": "z2c"}.get(direction, direction)
    return _real_apply(x, route, other, out_rows)


_real_roll = T.roll_labels


def _roll_uses_padded_end(ids, cu_padded, cu_real, total, max_shift, fill=0):
    return _real_roll(ids, cu_padded, None, total, max_shift, fill)


def _roll_off_by_one(ids, cu_padded, cu_real, total, max_shift, fill=0):
    shifted, mask = _real_roll(ids, cu_padded, cu_real, total, max_shift, fill)
    p = [int(v) for v in cu_padded]
    r = p if cu_real is None else [int(v) for v in cu_real]
    ids = np.asarray(ids, dtype=np.int64)
    for s in range(len(p) - 1):        # lets shift 1 reach one token past the document end
        e = p[s] + r[s + 1] - r[s]
        if e - 1 >= p[s] and e < total:
            shifted[0, e - 1] = ids[e]
            mask[1, e - 1] = 1
    return shifted, mask


def _check_monotone_skipped(cu, cp, total):
    b = [int(v) for v in np.asarray(cu).reshape(-1)]
    if b[0] != 0:
        raise T.OracleInputError("CU_START", "")
    if b[-1] != total:
        raise T.OracleInputError("CU_TOTAL", "")
    for i in range(len(b) - 1):
        if (b[i + 1] - b[i]) % (2 * cp):
            raise T.OracleInputError("CU_DIVISIBLE", "")
    return b


_real_pack = T.pack_batch


def _pack_eod_starts_next(tokens, pad_id, eod_id, align, capacity, max_docs, pad_value):
    # EOD opens the next document instead of closing its own
    rows = np.asarray(tokens, dtype=np.int64)
    shifted = rows.copy()
    for b in range(rows.shape[0]):
        for s in range(rows.shape[1] - 1, 0, -1):
            if rows[b, s - 1] == eod_id and rows[b, s] != pad_id:
                shifted[b, s - 1], shifted[b, s] = rows[b, s], rows[b, s - 1]
    return _real_pack(shifted, pad_id, eod_id, align, capacity, max_docs, pad_value)


def _pack_drops_trailing(tokens, pad_id, eod_id, align, capacity, max_docs, pad_value):
    rows = np.asarray(tokens, dtype=np.int64).copy()
    for b in range(rows.shape[0]):
        eods = np.flatnonzero(rows[b] == eod_id)
        cut = eods[-1] + 1 if eods.size else 0
        rows[b, cut:] = pad_id
    return _real_pack(rows, pad_id, eod_id, align, capacity, max_docs, pad_value)


def _pack_valid_end_at_first_pad(tokens, pad_id, eod_id, align, capacity, max_docs, pad_value):
    rows = np.asarray(tokens, dtype=np.int64).copy()
    for b in range(rows.shape[0]):
        pads = np.flatnonzero(rows[b] == pad_id)
        if pads.size:
            rows[b, pads[0]:] = pad_id
    return _real_pack(rows, pad_id, eod_id, align, capacity, max_docs, pad_value)


_real_roll_at = T.roll_valid_at


def _roll_at_inclusive_end(cu_padded, cu_real, token, shift):   # t + j <= e instead of t + j < e
    return _real_roll_at(cu_padded, cu_real, token, shift - 1) if shift > 0 else _real_roll_at(
        cu_padded, cu_real, token, shift)


def _roll_at_padded_end(cu_padded, cu_real, token, shift):      # real lengths ignored
    return _real_roll_at(cu_padded, None, token, shift)


MUTATIONS = {
    "single-position roll: label reaches one past the end": ("roll_valid_at", _roll_at_inclusive_end),
    "single-position roll: real lengths ignored": ("roll_valid_at", _roll_at_padded_end),
    "pack: EOD opens the next document": ("pack_batch", _pack_eod_starts_next),
    "pack: document after the last EOD dropped": ("pack_batch", _pack_drops_trailing),
    "pack: valid part ends at the first PAD": ("pack_batch", _pack_valid_end_at_first_pad),
    "back chunk index off by one": ("zigzag_rank_tokens", _zig_back_off_by_one),
    "back chunk before front chunk": ("zigzag_rank_tokens", _zig_back_first),
    "chunks of L/cp": ("zigzag_rank_tokens", _zig_chunk_by_cp),
    "contiguous ranks reversed": ("contiguous_rank_tokens", _contig_reversed),
    "swap directions exchanged": ("swap_rows", _swap_directions_exchanged),
    "route applied by its inverse": ("apply_route", _apply_gathers_by_the_inverse),
    "roll ignores real lengths": ("roll_labels", _roll_uses_padded_end),
    "label crosses the document end": ("roll_labels", _roll_off_by_one),
    "monotone check dropped": ("check_route_boundaries", _check_monotone_skipped),
}


@contextlib.contextmanager
def planted(name, fn):
    orig_t, orig_pkg = getattr(T, name), getattr(oracle, name)
    setattr(T, name, fn)
    setattr(oracle, name, fn)
    try:
        yield
    finally:
        setattr(T, name, orig_t)
        setattr(oracle, name, orig_pkg)


def run_pins():
    """Run the pins; return the names of those that fail."""
    worked = read_golden("p3_worked_example.txt")
    checks = [
        ("padding", lambda: P.test_worked_example_padding_reproduces_printed_boundaries(worked)),
        ("zigzag", lambda: P.test_worked_example_zigzag_indices(worked)),
        ("contiguous", lambda: P.test_worked_example_contiguous_indices(worked)),
        ("swap", lambda: P.test_worked_example_swap_gives_printed_rank_tokens(worked)),
        ("mask", lambda: P.test_worked_example_valid_mask_and_count(worked)),
        ("labels", lambda: P.test_worked_example_labels(worked)),
        ("single", P.test_single_document_example),
        ("runs", lambda: [P.test_hand_derived_runs_and_split(c) for c in ("worked", "tiny", "single")]),
        ("validation", lambda: P.test_validation_kinds([0, 8, 4, 16], 2, 16, "CU_MONOTONE")),
        ("roll kinds", lambda: P.test_roll_validation_kinds([0, 4, 8], [0, 5, 6], 8, "REAL_GT_PADDED")),
        ("brute force", lambda: [BF.test_zigzag_matches_sort_key_and_closed_form(cp) for cp in (2, 3)]),
        ("a2a", lambda: BF.test_emulated_all_to_all_matches_global_swap(2)),
        ("np.roll", BF.test_roll_matches_per_document_numpy_roll),
        ("single-position roll", BF.test_single_position_roll_form_matches_the_batch_form),
        ("no crossing", lambda: BF.test_roll_counts_and_no_crossing(1)),
        ("pack example", lambda: P.test_pack_reproduces_the_worked_example(worked)),
        ("pack budget", P.test_pack_budget_and_empty_slots),
        ("pack corners", lambda: [P.test_pack_corner_cases(r, d) for r, d in (
            (["a_bE__"], ["a_bE"]), (["aEbc_"], ["aE", "bc"]), (["EE_", "a__"], ["E", "E", "a"]))]),
    ]
    failed = []
    for name, fn in checks:
        try:
            fn()
        except (Exception, pytest.fail.Exception):  # assertion, pytest.raises miss, or an oracle error
            failed.append(name)
    return failed


def test_pins_pass_on_the_real_oracle():
    assert run_pins() == []


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_each_planted_mistake_is_caught(mutation):
    name, fn = MUTATIONS[mutation]
    with planted(name, fn):
        failed = run_pins()
    assert failed, f"no pin caught: {mutation}"
