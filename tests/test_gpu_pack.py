"""Device-side packing against the oracle, and the whole sync-free chain.

thd_pack turns [batch, seq] token rows into one padded stream and its
boundary lists ("Packed Sequence 与上下文并行" §2.2 steps (1)-(3)); the outputs
must equal the oracle's pack exactly, over rows with EOD tokens anywhere,
all-PAD rows, PAD inside documents and rows ending in EOD.  Then pack -> route
build -> zigzag roll -> batched swap runs with shapes fixed on the host and
must equal the oracle's pack -> roll -> c->z swap.
"""

import time

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import CODE_OF_KIND, dev_i32, dev_i64, say

pytestmark = pytest.mark.gpu

PAD, EOD = 0, 1


@pytest.fixture(scope="module")
def thd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_packed_sequence_amd as thd
    return thd


def test_pack_worked_example(thd, golden):
    import torch
    g = golden("p3_worked_example.txt")
    rows = np.array([[ord(c) for c in g["sample0"]], [ord(c) for c in g["sample1"]]], dtype=np.int64)
    packed, cu_real, cu_pad, status = thd.pack(dev_i64(rows), ord("_"), ord("E"), 4, 16, 3, ord("P"))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert "".join(chr(v) for v in packed.cpu().numpy()) == "".join(g["tokens"])
    assert cu_real.cpu().numpy().tolist()[:4] == [int(v) for v in g["cu_seqlens"]]
    assert cu_pad.cpu().numpy().tolist()[:4] == [int(v) for v in g["cu_seqlens_padded"]]


CASES = [
    # seed, batch, seq, eod_rate, pad_tail_max, inner_pad_rate, align, capacity_slack, max_docs_slack
    (0, 4, 64, 0.05, 16, 0.0, 4, 0, 0),
    (1, 8, 1000, 0.01, None, 0.02, 8, 64, 5),
    (2, 1, 4096, 0.002, 100, 0.0, 16, 512, 1),
    (3, 33, 300, 0.03, None, 0.05, 2, 2, 0),
    (4, 3, 2500, 0.0, 50, 0.0, 64, 128, 3),        # no EOD at all: one document per non-empty row
    (5, 2, 3000, 0.3, 10, 0.0, 4, 0, 0),           # EOD-dense: many one- and two-token documents
    (6, 1200, 17, 0.1, None, 0.1, 8, 1000, 10),    # many short rows
    (7, 2, 3072, 0.001, 1024, 0.0, 512, 3, 2),      # rows of whole 1024-token chunks, wide alignment
    (8, 3, 2048, 0.0, 1, 0.0, 3, 5, 1),             # one document per row crossing chunks, odd alignment
    (9, 3000, 1500, 0.002, 300, 0.01, 8, 10, 5),    # 6000 chunks: the scan carries across six passes
]


def test_pack_chunk_boundaries(thd):
    # EODs and valid ends on and next to the 1024-token chunk edges, where
    # a document's start and end fall in different chunks.
    import torch
    seq = 4096
    rows = np.full((6, seq), 5, dtype=np.int64)
    for r, (eods, valid_end) in enumerate([([1023], 2048), ([1024], 1025), ([1022, 1023, 1024, 2047], 4096),
                                           ([], 1024), ([0, 4095], 4096), ([3071], 3072)]):
        rows[r, valid_end:] = PAD
        rows[r, eods] = EOD
    align, max_docs = 8, 20
    capacity = 8 * 4096 + 64
    want = O.pack_batch(rows, PAD, EOD, align, capacity, max_docs, -3)
    packed, cu_real, cu_pad, status = thd.pack(dev_i64(rows), PAD, EOD, align, capacity, max_docs, -3)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(packed.cpu().numpy(), want[0])
    assert np.array_equal(cu_real.cpu().numpy(), want[1])
    assert np.array_equal(cu_pad.cpu().numpy(), want[2])


@pytest.mark.parametrize("case", CASES, ids=[f"seed{c[0]}" for c in CASES])
def test_pack_random_rows(thd, case):
    import torch
    seed, batch, seq, eod_rate, tail, inner, align, cap_slack, doc_slack = case
    rows = W.token_rows(seed, batch, seq, PAD, EOD, eod_rate, tail, inner)
    # size the budget from the oracle's own document list (a host-side choice)
    _, cu_r, cu_p = O.pack_batch(rows, PAD, EOD, align, batch * seq * align, batch * seq + 1, -9)
    n_docs = int(np.count_nonzero(np.diff(cu_r) > 0))   # documents have real tokens, the pad slot none
    used = int(cu_p[n_docs])
    capacity = used + cap_slack * align
    max_docs = n_docs + doc_slack
    say("pack", case, "docs", n_docs, "capacity", capacity)
    want = O.pack_batch(rows, PAD, EOD, align, capacity, max_docs, -9)
    packed, cu_real, cu_pad, status = thd.pack(dev_i64(rows), PAD, EOD, align, capacity, max_docs, -9)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(packed.cpu().numpy(), want[0])
    assert np.array_equal(cu_real.cpu().numpy(), want[1])
    assert np.array_equal(cu_pad.cpu().numpy(), want[2])


@pytest.mark.parametrize("max_docs,capacity,kind", [(1, 16, "PACK_DOCS"), (3, 12, "PACK_CAPACITY")])
def test_pack_overflow_writes_nothing(thd, golden, max_docs, capacity, kind):
    import torch
    g = golden("p3_worked_example.txt")
    rows = np.array([[ord(c) for c in g["sample0"]], [ord(c) for c in g["sample1"]]], dtype=np.int64)
    with pytest.raises(O.OracleInputError) as e:
        O.pack_batch(rows, ord("_"), ord("E"), 4, capacity, max_docs, 0)
    assert e.value.kind == kind
    nbytes = thd.thd_pack_workspace_bytes(2, 8)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    packed = torch.full((capacity,), -5, dtype=torch.int64, device="cuda")
    cu_real = torch.full((max_docs + 2,), -5, dtype=torch.int32, device="cuda")
    cu_pad = torch.full((max_docs + 2,), -5, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert thd.thd_pack(dev_i64(rows), 2, 8, ord("_"), ord("E"), 4, capacity, max_docs, 0, ws, nbytes, packed,
                        cu_real, cu_pad, status) == thd.THD_OK
    torch.cuda.synchronize()
    assert int(status.item()) == {"PACK_DOCS": thd.THD_ERR_PACK_DOCS, "PACK_CAPACITY": thd.THD_ERR_PACK_CAPACITY}[kind]
    assert (packed == -5).all() and (cu_real == -5).all() and (cu_pad == -5).all()


def test_pack_empty_batch(thd):
    import torch
    rows = np.zeros((3, 5), dtype=np.int64)            # all PAD: no documents
    packed, cu_real, cu_pad, status = thd.pack(dev_i64(rows), PAD, EOD, 4, 8, 2, 7)
    torch.cuda.synchronize()
    want = O.pack_batch(rows, PAD, EOD, 4, 8, 2, 7)
    assert int(status.item()) == 0
    assert np.array_equal(packed.cpu().numpy(), want[0])
    assert np.array_equal(cu_real.cpu().numpy(), want[1]) and np.array_equal(cu_pad.cpu().numpy(), want[2])


@pytest.mark.parametrize("cp,seed", [(2, 10), (4, 11), (8, 12)])
def test_pack_route_roll_swap_chain(thd, cp, seed):
    # Rows -> pack -> route -> roll in zigzag order + multi-key swap, every
    # shape fixed on the host (budget T, max_docs + 1 slots); then the same
    # chain on the oracle.  A spin kernel holds the stream while it is
    # enqueued: no call may wait for the GPU.
    import torch
    batch, seq, align = 8, 2000, 2 * cp * 4
    rows = W.token_rows(seed, batch, seq, PAD, EOD, 0.004, 400, 0.0)
    max_docs = 200
    capacity = ((batch * seq) // align + max_docs + 1) * align
    want_packed, want_cu, want_cup = O.pack_batch(rows, PAD, EOD, align, capacity, max_docs, PAD)
    n_slots = max_docs + 1
    say("chain", cp, "capacity", capacity)

    tokens = dev_i64(rows)
    nbytes = thd.thd_pack_workspace_bytes(batch, seq)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    packed = torch.empty(capacity, dtype=torch.int64, device="cuda")
    cu_real = torch.empty(max_docs + 2, dtype=torch.int32, device="cuda")
    cu_pad = torch.empty(max_docs + 2, dtype=torch.int32, device="cuda")
    pstatus = torch.empty(1, dtype=torch.int32, device="cuda")
    route = thd.Route(n_slots, cp, capacity)
    shifted = torch.empty((2, capacity), dtype=torch.int64, device="cuda")
    mask = torch.empty((3, capacity), dtype=torch.uint8, device="cuda")
    rstatus = torch.empty(1, dtype=torch.int32, device="cuda")
    zig_tokens = torch.empty_like(packed)
    pos = torch.arange(capacity, dtype=torch.int64, device="cuda")
    zig_pos = torch.empty_like(pos)
    torch.cuda.synchronize()

    gate = torch.cuda.Event()
    torch.cuda._sleep(int(3e8))
    gate.record()
    t0 = time.perf_counter()
    thd.thd_pack(tokens, batch, seq, PAD, EOD, align, capacity, max_docs, PAD, ws, nbytes, packed, cu_real, cu_pad,
                 pstatus)
    thd.thd_build_route(route.handle, cu_pad, n_slots, cp, capacity)
    thd.thd_roll_labels_zigzag(route.handle, packed, cu_pad, cu_real, n_slots, capacity, 2, -1, shifted, mask,
                               rstatus)
    thd.thd_swap_batch(route.handle, thd.C2Z, [packed, pos], [zig_tokens, zig_pos], [8, 8], capacity)
    enqueue = time.perf_counter() - t0
    waited = gate.query()
    torch.cuda.synchronize()
    say(f"chain enqueue {enqueue * 1e3:.2f} ms")
    assert not waited, "a call in the chain waited for the GPU"
    assert int(pstatus.item()) == 0 and int(rstatus.item()) == 0 and route.status() == 0
    assert np.array_equal(packed.cpu().numpy(), want_packed)
    ws_, wm_ = O.roll_labels(want_packed, want_cup, want_cu, capacity, 2, -1)
    for k in range(2):
        assert np.array_equal(shifted[k].cpu().numpy(), O.swap_rows(ws_[k], want_cup, cp, capacity, "c2z"))
    for k in range(3):
        assert np.array_equal(mask[k].cpu().numpy(), O.swap_rows(wm_[k], want_cup, cp, capacity, "c2z"))
    assert np.array_equal(zig_tokens.cpu().numpy(), O.swap_rows(want_packed, want_cup, cp, capacity, "c2z"))
    assert np.array_equal(zig_pos.cpu().numpy(), O.layout_tokens(want_cup, cp, capacity, O.ZIGZAG))


@pytest.mark.parametrize("batch,seq,align", [(16, 8192, 8), (16, 16384, 32), (16, 65536, 8)])
def test_pack_at_bench_sizes(thd, batch, seq, align):
    # The inputs and launch the bench times for the 128K, full and 1M
    # batches ([16, T/16] rows, 256 document slots), compared in full.
    import torch
    max_docs = 256
    rows = W.token_rows(7, batch, seq, PAD, EOD, 1.0 / 4096, 512)
    capacity = ((batch * seq) // align + max_docs + 1) * align
    say("pack bench size", batch, seq, align)
    want = O.pack_batch(rows, PAD, EOD, align, capacity, max_docs, PAD)
    packed, cu_real, cu_pad, status = thd.pack(dev_i64(rows), PAD, EOD, align, capacity, max_docs, PAD)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(packed.cpu().numpy(), want[0])
    assert np.array_equal(cu_real.cpu().numpy(), want[1])
    assert np.array_equal(cu_pad.cpu().numpy(), want[2])
