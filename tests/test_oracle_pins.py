"""Pins of the CPU oracle to values the pages print (CPU only).

Fixtures under tests/golden/ carry the page citations.  Every test here fails
for the plausible mistakes in the oracle: a wrong chunk index for the back
chunk, front/back order swapped, the two swap directions exchanged, labels that
run into the next document or into pads.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from conftest import read_golden, read_run_cases


def _ints(v):
    return [int(x) for x in v]


@pytest.fixture(scope="module")
def worked():
    return read_golden("p3_worked_example.txt")


def test_worked_example_padding_reproduces_printed_boundaries(worked):
    # §3.3: per-document padding to align_size gives the printed padded boundaries.
    seqlens = _ints(worked["seqlens"])
    align = int(worked["align_size"][0])
    padded = W.pad_to_multiple(seqlens, align)
    assert padded.tolist() == _ints(worked["padded_seqlens"])
    assert (padded - np.asarray(seqlens)).tolist() == _ints(worked["padding"])
    assert W.cumulative(padded).tolist() == _ints(worked["cu_seqlens_padded"])
    assert W.cumulative(seqlens).tolist() == _ints(worked["cu_seqlens"])


def test_worked_example_zigzag_indices(worked):
    cu = _ints(worked["cu_seqlens_padded"])
    assert O.zigzag_rank_tokens(cu, 2, 0).tolist() == _ints(worked["rank0_index"])
    assert O.zigzag_rank_tokens(cu, 2, 1).tolist() == _ints(worked["rank1_index"])


def test_worked_example_contiguous_indices(worked):
    assert O.contiguous_rank_tokens(16, 2, 0).tolist() == _ints(worked["ulysses_rank0"])
    assert O.contiguous_rank_tokens(16, 2, 1).tolist() == _ints(worked["ulysses_rank1"])


def test_worked_example_swap_gives_printed_rank_tokens(worked):
    # The packed stream is the contiguous (natural) order; c->z must hand each
    # rank exactly the tokens printed for it in §3.6, and z->c must undo it.
    cu = _ints(worked["cu_seqlens_padded"])
    stream = np.frombuffer("".join(worked["tokens"]).encode(), dtype=np.uint8).copy()
    z = O.swap_rows(stream, cu, 2, 16, "c2z")
    got0 = z[:8].tobytes().decode()
    got1 = z[8:].tobytes().decode()
    assert got0 == "".join(worked["rank0_tokens"])
    assert got1 == "".join(worked["rank1_tokens"])
    back = O.swap_rows(z, cu, 2, 16, "z2c")
    assert back.tobytes() == stream.tobytes()
    # Feeding the packed stream as if it were zigzag must NOT reproduce the page:
    # catches a swap with its two directions exchanged.
    wrong = O.swap_rows(stream, cu, 2, 16, "z2c")
    assert wrong[:8].tobytes().decode() != "".join(worked["rank0_tokens"])


def test_worked_example_valid_mask_and_count(worked):
    cu_pad = _ints(worked["cu_seqlens_padded"])
    cu = _ints(worked["cu_seqlens"])
    ids = np.arange(16, dtype=np.int64)
    shifted, mask = O.roll_labels(ids, cu_pad, cu, 16, 2)
    assert mask[0].tolist() == _ints(worked["valid_mask"])
    assert int(mask[0].sum()) == int(worked["valid_total"][0])
    assert int(mask[0].sum()) == sum(_ints(worked["valid_token_nums"]))
    # per-rank masks of §3.6 = the valid mask moved with the c->z swap
    zmask = O.swap_rows(mask[0], cu_pad, 2, 16, "c2z")
    assert zmask[:8].tolist() == _ints(worked["rank0_valid_mask"])
    assert zmask[8:].tolist() == _ints(worked["rank1_valid_mask"])


def test_worked_example_labels(worked):
    # Next-token labels inside each document of §3.4; the last real token of a
    # document and every pad get no label (fill = -1 here).  Hand-derived from
    # the printed stream: b c E - | e E - - | g h i j E - - -
    cu_pad = _ints(worked["cu_seqlens_padded"])
    cu = _ints(worked["cu_seqlens"])
    stream = np.frombuffer("".join(worked["tokens"]).encode(), dtype=np.uint8).astype(np.int64)
    shifted, mask = O.roll_labels(stream, cu_pad, cu, 16, 2, fill=-1)
    want = "b c E - e E - - g h i j E - - -".split()
    got = ["-" if v == -1 else chr(v) for v in shifted[0].tolist()]
    assert got == want
    assert mask[1].tolist() == [1, 1, 1, 0, 1, 1, 0, 0, 1, 1, 1, 1, 1, 0, 0, 0]
    assert int(mask[1].sum()) == 10
    assert int(mask[2].sum()) == 7
    # shift 2 (MTP depth 1 target): c E - - | E - - - | h i j E - - - -
    got2 = ["-" if v == -1 else chr(v) for v in shifted[1].tolist()]
    assert got2 == "c E - - E - - - h i j E - - - -".split()


def test_single_document_example():
    g = read_golden("p3_single_document.txt")
    cu = _ints(g["cu_seqlens_padded"])
    cp = int(g["cp"][0])
    assert O.zigzag_rank_tokens(cu, cp, 0).tolist() == _ints(g["rank0_index"])
    assert O.zigzag_rank_tokens(cu, cp, 1).tolist() == _ints(g["rank1_index"])


@pytest.mark.parametrize("case", ["worked", "tiny", "single"])
def test_hand_derived_runs_and_split(case):
    c = read_run_cases("derived_runs.txt")[case]
    cp = c["cp"][0]
    cu = c["cu_padded"]
    total = cu[-1]
    share = total // cp
    route = O.build_route(cu, cp, total)
    assert route["split"].reshape(-1).tolist() == c["split"]
    runs = O.canonical_runs(route)
    want = [[sr * share + sl, dr * share + dl, n] for sr, sl, dr, dl, n in c["runs"]]
    assert runs.tolist() == want


def test_cp1_is_identity():
    # Relax PR #273 §2.6: cp == 1 short-circuits; the output is the input object.
    x = np.arange(40, dtype=np.uint16).reshape(10, 4)
    assert O.swap_rows(x, [0, 3, 10], 1, 10, "z2c") is x
    assert O.swap_rows(x, [0, 3, 10], 1, 10, "c2z") is x
    assert O.build_route([0, 3, 10], 1, 10)["identity"]


def test_cp1_layouts_coincide():
    # With one rank, both slices hand every token to rank 0 in natural order.
    cu = [0, 2, 6, 6, 10]
    assert O.zigzag_rank_tokens(cu, 1, 0).tolist() == list(range(10))
    assert O.contiguous_rank_tokens(10, 1, 0).tolist() == list(range(10))


@pytest.mark.parametrize("cu,cp,total,kind", [
    ([0, 6, 16], 2, 16, "CU_DIVISIBLE"),        # 6 not a multiple of 4
    ([1, 8, 16], 2, 16, "CU_START"),
    ([0, 8, 4, 16], 2, 16, "CU_MONOTONE"),
    ([0, 8, 16], 2, 24, "CU_TOTAL"),
    # precedence: start beats everything, monotone beats total and divisibility
    ([2, 1, 7], 2, 9, "CU_START"),
    ([0, 9, 3, 12], 2, 16, "CU_MONOTONE"),
    ([0, 6, 12], 2, 16, "CU_TOTAL"),
])
def test_validation_kinds(cu, cp, total, kind):
    with pytest.raises(O.OracleInputError) as e:
        O.build_route(cu, cp, total)
    assert e.value.kind == kind
    assert isinstance(e.value, ValueError)


def test_invalid_direction():
    with pytest.raises(O.OracleInputError) as e:
        O.swap_rows(np.zeros((8, 2), np.uint8), [0, 8], 2, 8, "sideways")
    assert e.value.kind == "DIRECTION"


@pytest.mark.parametrize("cu_pad,cu_real,total,kind", [
    ([1, 4, 8], [0, 3, 6], 8, "CU_START"),
    ([0, 4, 8], [1, 3, 6], 8, "CU_START"),
    ([0, 4, 2, 8], [0, 3, 3, 6], 8, "CU_MONOTONE"),
    ([0, 4, 8], [0, 3, 2], 8, "CU_MONOTONE"),
    ([0, 4, 8], [0, 3, 6], 12, "CU_TOTAL"),
    ([0, 4, 8], [0, 5, 6], 8, "REAL_GT_PADDED"),
])
def test_roll_validation_kinds(cu_pad, cu_real, total, kind):
    with pytest.raises(O.OracleInputError) as e:
        O.roll_labels(np.zeros(total, np.int64), cu_pad, cu_real, total, 1)
    assert e.value.kind == kind


def test_tiny_workload_matches_hand_derivation():
    w = W.make("tiny")
    assert w.cu_padded.tolist() == [0, 8, 20, 24]
    z0 = O.zigzag_rank_tokens(w.cu_padded, 2, 0).tolist()
    z1 = O.zigzag_rank_tokens(w.cu_padded, 2, 1).tolist()
    assert z0 == [0, 1, 6, 7, 8, 9, 10, 17, 18, 19, 20, 23]
    assert z1 == [2, 3, 4, 5, 11, 12, 13, 14, 15, 16, 21, 22]


# ---- packing ("Packed Sequence 与上下文并行" §2.2, worked example §3.1-§3.4) ----

def _encode(chars):
    return [ord(c) for c in chars]


PAD, EOD = ord("_"), ord("E")


def test_pack_reproduces_the_worked_example(worked):
    rows = [_encode(worked["sample0"]), _encode(worked["sample1"])]
    align = int(worked["align_size"][0])
    packed, cu_real, cu_pad = O.pack_batch(rows, PAD, EOD, align, 16, 3, ord("P"))
    assert "".join(chr(v) for v in packed) == "".join(worked["tokens"])
    assert cu_real[:4].tolist() == _ints(worked["cu_seqlens"])
    assert cu_pad[:4].tolist() == _ints(worked["cu_seqlens_padded"])
    # one trailing slot (empty here: the documents fill the budget exactly)
    assert cu_real.tolist()[4:] == [13] and cu_pad.tolist()[4:] == [16]
    _, mask = O.roll_labels(packed, cu_pad, cu_real, 16, 1)
    assert mask[0].tolist() == _ints(worked["valid_mask"])


def test_pack_budget_and_empty_slots():
    # Room for 5 documents in 24 tokens: 3 documents (12 padded tokens), a
    # trailing pad slot of 12, two empty slots.
    rows = [_encode("abE_____"), _encode("cdeEf___")]
    packed, cu_real, cu_pad = O.pack_batch(rows, PAD, EOD, 4, 24, 5, -1)
    assert cu_real.tolist() == [0, 3, 7, 8, 8, 8, 8]
    assert cu_pad.tolist() == [0, 4, 8, 12, 24, 24, 24]
    assert packed.tolist()[:12] == _encode("abE") + [-1] + _encode("cdeE") + _encode("f") + [-1, -1, -1]
    assert (packed[12:] == -1).all()


@pytest.mark.parametrize("rows,want_docs", [
    (["____"], []),                                   # an all-pad row has no document
    (["a_bE__"], ["a_bE"]),                           # PAD inside the valid part stays in the document
    (["abE"], ["abE"]),                               # a row ending in EOD: no empty trailing document
    (["aEbc_"], ["aE", "bc"]),                        # the last document has no EOD
    (["abcd"], ["abcd"]),                             # one document fills the row
    (["EE_", "a__"], ["E", "E", "a"]),                # back-to-back EODs; rows stay separate
])
def test_pack_corner_cases(rows, want_docs):
    packed, cu_real, cu_pad = O.pack_batch([_encode(r) for r in rows], PAD, EOD, 2, 32, 8, 0)
    n = len(want_docs)
    lens = [len(d) for d in want_docs]
    assert np.diff(cu_real[:n + 1]).tolist() == lens
    assert np.diff(cu_pad[:n + 1]).tolist() == [v + v % 2 for v in lens]
    for k, d in enumerate(want_docs):
        assert "".join(chr(v) for v in packed[cu_pad[k]:cu_pad[k] + len(d)]) == d


@pytest.mark.parametrize("max_docs,capacity,kind", [(1, 16, "PACK_DOCS"), (3, 12, "PACK_CAPACITY")])
def test_pack_overflow(worked, max_docs, capacity, kind):
    rows = [_encode(worked["sample0"]), _encode(worked["sample1"])]
    with pytest.raises(O.OracleInputError) as e:
        O.pack_batch(rows, PAD, EOD, 4, capacity, max_docs, 0)
    assert e.value.kind == kind
