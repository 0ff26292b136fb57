"""thd_pack_noalloc (the pack for callers that cannot allocate) against thd_pack.

The same rows go through thd_pack with a workspace of its own and through
thd_pack_noalloc, which works in the library's static device scratch; every
output must be equal element for element.  Two calls in a row, the second on a
smaller batch, so the scratch holds the first call's contents when the second
starts; the first at the largest batch the scratch admits.  A batch one chunk
larger is refused on the host before any device work.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import dev_i64, say

pytestmark = pytest.mark.gpu

PAD, EOD = 0, 1


@pytest.fixture(scope="module")
def thd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_packed_sequence_amd as thd
    return thd


def _outputs(torch, capacity, max_docs):
    packed = torch.full((capacity,), -7, dtype=torch.int64, device="cuda")
    cu_real = torch.full((max_docs + 2,), -7, dtype=torch.int32, device="cuda")
    cu_pad = torch.full((max_docs + 2,), -7, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    return packed, cu_real, cu_pad, status


def _both(thd, torch, rows, align, capacity, max_docs, pad_value):
    batch, seq = rows.shape
    tokens = dev_i64(rows)
    nbytes = thd.thd_pack_workspace_bytes(batch, seq)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ref = _outputs(torch, capacity, max_docs)
    thd.thd_pack(tokens, batch, seq, PAD, EOD, align, capacity, max_docs, pad_value, ws, nbytes, *ref)
    got = _outputs(torch, capacity, max_docs)
    thd.thd_pack_noalloc(tokens, batch, seq, PAD, EOD, align, capacity, max_docs, pad_value, *got)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got]


def _largest_seq(thd, batch):
    """Largest row length (a whole number of 1024-token chunks) whose pack
    fits the static scratch."""
    seq = 1024
    while thd.thd_pack_workspace_bytes(batch, seq + 1024) <= thd.THD_PACK_STATIC_BYTES:
        seq += 1024
    return seq


def test_noalloc_pack_matches_pack_twice_in_a_row(thd):
    import torch
    # first call: the largest batch of 2 rows the scratch admits (three
    # launches: more chunks than one scan pass covers)
    batch = 2
    seq = _largest_seq(thd, batch)
    assert thd.thd_pack_workspace_bytes(batch, seq) <= thd.THD_PACK_STATIC_BYTES
    rows = W.token_rows(70, batch, seq, PAD, EOD, 1.0 / 5000, 2048)
    align, max_docs = 8, 16384
    capacity = ((batch * seq) // align + max_docs + 1) * align
    say("noalloc pack, first call", batch, seq, "tokens", batch * seq, "capacity", capacity)
    ref, got = _both(thd, torch, rows, align, capacity, max_docs, -1)
    assert ref[3][0] == thd.THD_OK
    for r, g in zip(ref, got):
        assert np.array_equal(r, g)

    # second call: a smaller batch (one fused launch pair), through the same
    # scratch still holding the first call's chunk records; also against the
    # oracle
    rows2 = W.token_rows(71, 5, 3000, PAD, EOD, 0.01, 500, 0.01)
    _, cu_r, cu_p = O.pack_batch(rows2, PAD, EOD, 4, 5 * 3000 * 4, 5 * 3000 + 1, -2)
    n_docs = int(np.count_nonzero(np.diff(cu_r) > 0))
    capacity2 = int(cu_p[n_docs]) + 16
    max_docs2 = n_docs + 3
    say("noalloc pack, second call", rows2.shape, "docs", n_docs)
    ref2, got2 = _both(thd, torch, rows2, 4, capacity2, max_docs2, -2)
    assert ref2[3][0] == thd.THD_OK
    for r, g in zip(ref2, got2):
        assert np.array_equal(r, g)
    want = O.pack_batch(rows2, PAD, EOD, 4, capacity2, max_docs2, -2)
    for w_, g in zip(want, got2[:3]):
        assert np.array_equal(w_, g)


def test_noalloc_pack_refuses_a_batch_beyond_its_scratch(thd):
    import torch
    batch = 2
    seq = _largest_seq(thd, batch) + 1024
    assert thd.thd_pack_workspace_bytes(batch, seq) > thd.THD_PACK_STATIC_BYTES
    tokens = torch.full((batch, seq), 5, dtype=torch.int64, device="cuda")
    capacity, max_docs = batch * seq + 64, 8
    outs = _outputs(torch, capacity, max_docs)
    with pytest.raises(thd.ThdError) as e:
        thd.thd_pack_noalloc(tokens, batch, seq, PAD, EOD, 8, capacity, max_docs, 0, *outs)
    assert e.value.code == thd.THD_ERR_CAPACITY
    torch.cuda.synchronize()
    for t in outs:
        assert (t == -7).all()  # nothing was launched
