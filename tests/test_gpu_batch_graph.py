"""Multi-tensor swap, roll written in zigzag order, and HIP-graph capture.

* thd_swap_batch moves the per-token streams of a packed batch (token ids,
  labels, loss mask, position ids, valid mask) and an activation through one
  route in one launch ("Packed Sequence 与上下文并行" §2.4 slices every key
  with the same index); each output must equal the oracle's swap of that
  tensor byte for byte.
* thd_roll_labels_zigzag must equal the oracle's roll followed by the oracle's
  c->z swap of every output stream.
* A HIP graph capturing build + swaps + roll replays to the eager results,
  and picks up new boundaries written into the captured buffer (the route is
  a device-resident capture input).
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import dev_i32, dev_i64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def thd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_packed_sequence_amd as thd
    return thd


def batch_keys(w, rng):
    """Per-token streams of a packed batch plus one activation (host arrays)."""
    t = w.total
    return {
        "tokens": w.ids(),
        "labels": rng.integers(-1, 32000, size=t, dtype=np.int64),
        "loss_mask": rng.integers(0, 2, size=t, dtype=np.uint8),
        "position_ids": rng.integers(0, 65536, size=t, dtype=np.int64),
        "valid_mask": rng.integers(0, 2, size=t, dtype=np.uint8),
        "fp32_pair": rng.standard_normal((t, 2), dtype=np.float32),
        "int64_pair": rng.integers(-2 ** 62, 2 ** 62, size=(t, 2), dtype=np.int64),   # one 16-byte unit per row
        "hidden": w.rows_host().view(np.int16),      # bf16 bit patterns
        "wide": rng.integers(0, 256, size=(t, 4624), dtype=np.uint8),   # rows split into two slices
    }


@pytest.mark.parametrize("seed,cp,docs,max_chunk,n_empty", [
    (0, 2, 9, 40, 0), (1, 4, 40, 64, 3), (2, 8, 25, 20, 8), (3, 3, 200, 6, 30), (4, 16, 12, 9, 4)])
def test_swap_batch_matches_per_tensor_oracle(thd, seed, cp, docs, max_chunk, n_empty):
    import torch
    w = W.random_packed(seed, cp, docs, max_chunk, n_empty, row_shape=(2, 24))
    cu, total = w.cu_padded, w.total
    say("batch", seed, cp, "T", total)
    route = thd.Route(w.n_slots, cp, total)
    route.build(dev_i32(cu), cp, total)
    keys = batch_keys(w, np.random.default_rng(seed))
    xs = [torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in keys.values()]
    for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
        outs = route.swap_many(xs, d)
        torch.cuda.synchronize()
        for (name, host), out in zip(keys.items(), outs):
            want = O.swap_rows(host, cu, cp, total, direction)
            assert np.array_equal(out.cpu().numpy().view(host.dtype), want), (name, direction)


def test_swap_batch_full_workload(thd):
    # The full micro-batch's per-token streams in one launch, plus the guard
    # that outputs land only where they belong (sentinel around each output).
    import torch
    w = W.make("full")
    cu, total, cp = w.cu_padded, w.total, w.cp
    route = thd.Route(w.n_slots, cp, total)
    route.build(dev_i32(cu), cp, total)
    rng = np.random.default_rng(9)
    keys = batch_keys(w, rng)
    keys.pop("hidden")
    keys.pop("wide")
    xs = [torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in keys.values()]
    pads = []
    outs = []
    for x in xs:
        nbytes = x.numel() * x.element_size()
        buf = torch.full((nbytes + 256,), 0xA5, dtype=torch.uint8, device="cuda")
        pads.append(buf)
        outs.append(buf[128:128 + nbytes].view(x.dtype).view(x.shape))
    rbs = [x.numel() * x.element_size() // total for x in xs]
    assert thd.thd_swap_batch(route.handle, thd.C2Z, xs, outs, rbs, total) == thd.THD_OK
    torch.cuda.synchronize()
    for (name, host), out, buf in zip(keys.items(), outs, pads):
        assert np.array_equal(out.cpu().numpy(), O.swap_rows(host, cu, cp, total, "c2z")), name
        b = buf.cpu().numpy()
        assert (b[:128] == 0xA5).all() and (b[-128:] == 0xA5).all(), name


def test_swap_batch_errors(thd):
    import torch
    route = thd.Route(4, 2, 32)
    route.build(dev_i32([0, 16, 32]), 2, 32)
    a = torch.zeros(32, 8, dtype=torch.uint8, device="cuda")
    b = torch.zeros(32, 8, dtype=torch.uint8, device="cuda")
    c = torch.zeros(32, 4, dtype=torch.uint8, device="cuda")
    for args, code in [
        ((route.handle, thd.Z2C, [a, b], [c, c], [8, 8], 32), thd.THD_ERR_ALIAS),       # two outputs overlap
        ((route.handle, thd.Z2C, [a, b], [b, c], [8, 8], 32), thd.THD_ERR_ALIAS),       # output over an input
        ((route.handle, 5, [a], [b], [8], 32), thd.THD_ERR_DIRECTION),
        ((route.handle, thd.Z2C, [a], [b], [8], 16), thd.THD_ERR_SHAPE),
        ((route.handle, thd.Z2C, [a], [b], [0], 32), thd.THD_ERR_ARG),
        ((route.handle, thd.Z2C, [a] * 17, [b] * 17, [8] * 17, 32), thd.THD_ERR_ARG),
    ]:
        with pytest.raises(thd.ThdError) as e:
            thd.thd_swap_batch(*args)
        assert e.value.code == code, args


@pytest.mark.parametrize("name", ["tiny", "gdn128k", "full"])
def test_roll_zigzag_matches_roll_then_slice(thd, name):
    import torch
    w = W.make(name)
    cu, total, cp = w.cu_padded, w.total, w.cp
    j = max(w.max_shift, 2)
    route = thd.Route(w.n_slots, cp, total)
    route.build(dev_i32(cu), cp, total)
    ids = w.ids()
    say("roll zigzag", name)
    shifted, mask, status = route.roll_labels_zigzag(dev_i64(ids), dev_i32(cu), dev_i32(w.cu_real), j, -1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    want_s, want_m = O.roll_labels(ids, cu, w.cu_real, total, j, -1)
    for k in range(j):
        assert np.array_equal(shifted[k].cpu().numpy(), O.swap_rows(want_s[k], cu, cp, total, "c2z")), k
    for k in range(j + 1):
        assert np.array_equal(mask[k].cpu().numpy(), O.swap_rows(want_m[k], cu, cp, total, "c2z")), k


def test_roll_zigzag_worked_example(thd, golden):
    # §3.6: each rank's valid mask after the slice, straight from the roll.
    import torch
    g = golden("p3_worked_example.txt")
    cu_pad = [int(v) for v in g["cu_seqlens_padded"]]
    cu = [int(v) for v in g["cu_seqlens"]]
    route = thd.Route(3, 2, 16)
    route.build(dev_i32(cu_pad), 2, 16)
    _, mask, status = route.roll_labels_zigzag(dev_i64(np.arange(16)), dev_i32(cu_pad), dev_i32(cu), 1, 0)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    m = mask[0].cpu().numpy().tolist()
    assert m[:8] == [int(v) for v in g["rank0_valid_mask"]]
    assert m[8:] == [int(v) for v in g["rank1_valid_mask"]]


def test_roll_zigzag_bad_route_writes_nothing(thd):
    import torch
    route = thd.Route(2, 2, 16)
    route.build(dev_i32([0, 6, 16]), 2, 16)           # length 6 not a multiple of 4
    shifted = torch.full((1, 16), -3, dtype=torch.int64, device="cuda")
    mask = torch.full((2, 16), 9, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    code = thd.thd_roll_labels_zigzag(route.handle, torch.arange(16, device="cuda"), dev_i32([0, 6, 16]), None, 2,
                                      16, 1, 0, shifted, mask, status)
    assert code == thd.THD_OK
    torch.cuda.synchronize()
    assert int(status.item()) == thd.THD_ERR_CU_DIVISIBLE
    assert (shifted == -3).all() and (mask == 9).all()
    with pytest.raises(thd.ThdError) as e:
        thd.thd_roll_labels_zigzag(route.handle, torch.arange(8, device="cuda"), dev_i32([0, 8]), None, 1, 8, 1, 0,
                                   shifted, mask, status)
    assert e.value.code == thd.THD_ERR_SHAPE
    # the same token count with another slot count is another batch too
    with pytest.raises(thd.ThdError) as e:
        thd.thd_roll_labels_zigzag(route.handle, torch.arange(16, device="cuda"), dev_i32([0, 16]), None, 1, 16, 1, 0,
                                   shifted, mask, status)
    assert e.value.code == thd.THD_ERR_SHAPE


def test_graph_capture_replays_build_swaps_and_roll(thd):
    # Capture one micro-batch (build, 8 layers x 2 swaps, zigzag roll) in a
    # HIP graph; replay it several times with eager work in between, and once
    # after writing different boundaries into the captured buffer.
    import torch
    wa = W.random_packed(500, 4, 30, 40, 2, pad_max=3, row_shape=(2048,), row_dtype="uint8")
    total, cp = wa.total, wa.cp
    # a second batch with the same token and slot counts: the documents reordered
    perm = np.random.default_rng(7).permutation(wa.n_slots)
    wb = W.Workload("reordered", 100, cp, W.cumulative(np.diff(wa.cu_padded)[perm]),
                    W.cumulative(np.diff(wa.cu_real)[perm]), (2048,), row_dtype="uint8", max_shift=1,
                    seed_extra=(501,))
    assert not np.array_equal(wb.cu_padded, wa.cu_padded)
    route = thd.Route(wa.n_slots, cp, total)
    cu = dev_i32(wa.cu_padded)
    cu_real = dev_i32(wa.cu_real)
    x = torch.from_numpy(wa.rows_host()).cuda()
    ids = dev_i64(wa.ids())
    a, b = torch.empty_like(x), torch.empty_like(x)
    shifted = torch.empty((2, total), dtype=torch.int64, device="cuda")
    mask = torch.empty((3, total), dtype=torch.uint8, device="cuda")
    status = torch.empty(1, dtype=torch.int32, device="cuda")
    n_slots = wa.n_slots

    def step(stream):
        thd.thd_build_route(route.handle, cu, n_slots, cp, total, stream)
        for _ in range(8):
            thd.thd_swap(route.handle, thd.Z2C, x, a, total, 2048, stream)
            thd.thd_swap(route.handle, thd.C2Z, a, b, total, 2048, stream)
        thd.thd_roll_labels_zigzag(route.handle, ids, cu, cu_real, n_slots, total, 2, 0, shifted, mask, status,
                                   stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s.cuda_stream)                          # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    def expect(w):
        want_a = O.swap_rows(w.rows_host(), w.cu_padded, cp, total, "z2c")
        ws, wm = O.roll_labels(w.ids(), w.cu_padded, w.cu_real, total, 2, 0)
        return want_a, [O.swap_rows(ws[k], w.cu_padded, cp, total, "c2z") for k in range(2)], \
            [O.swap_rows(wm[k], w.cu_padded, cp, total, "c2z") for k in range(3)]

    want_a, want_s, want_m = expect(wa)
    for rep in range(3):
        a.zero_(); b.zero_(); shifted.zero_(); mask.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("graph replay", rep)
        assert int(status.item()) == 0
        assert np.array_equal(a.cpu().numpy(), want_a)
        assert torch.equal(b, x)
        for k in range(2):
            assert np.array_equal(shifted[k].cpu().numpy(), want_s[k])
        for k in range(3):
            assert np.array_equal(mask[k].cpu().numpy(), want_m[k])
        _ = (x.float().sum() + 1).item()             # eager work between replays
    cu.copy_(dev_i32(wb.cu_padded))
    cu_real.copy_(dev_i32(wb.cu_real))
    x.copy_(torch.from_numpy(wb.rows_host()).cuda())
    ids.copy_(dev_i64(wb.ids()))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    want_a, want_s, want_m = expect(wb)
    assert np.array_equal(a.cpu().numpy(), want_a)
    for k in range(2):
        assert np.array_equal(shifted[k].cpu().numpy(), want_s[k])


def test_graph_capture_of_the_full_microbatch(thd):
    # The configured 48-layer micro-batch (cp 16, T = 262144, rows of 4 KiB):
    # route build, 48 x (z->c, c->z) and the zigzag label roll with MTP
    # depths 1..3 (shifts 1..4) captured in one HIP graph.  Replays with eager
    # work in between, then one replay after a second batch (same token and
    # slot counts, documents reordered, other rows and ids) is written into the
    # captured inputs; every replay is checked against the oracle.
    import torch
    wa = W.make("full")
    total, cp, n_slots, J = wa.total, wa.cp, wa.n_slots, wa.max_shift
    perm = np.random.default_rng(11).permutation(n_slots)
    wb = W.Workload("full-reordered", 101, cp, W.cumulative(np.diff(wa.cu_padded)[perm]),
                    W.cumulative(np.diff(wa.cu_real)[perm]), wa.row_shape, max_shift=J, layers=wa.layers,
                    seed_extra=(502,))
    assert not np.array_equal(wb.cu_padded, wa.cu_padded) and wb.total == total
    say("full micro-batch graph: T", total, "cp", cp, "layers", wa.layers)
    route = thd.Route(n_slots, cp, total)
    cu, cu_real = dev_i32(wa.cu_padded), dev_i32(wa.cu_real)
    ids = dev_i64(wa.ids())

    def rows_for(seed):
        g = torch.Generator(device="cuda").manual_seed(seed)
        v = torch.randn((total,) + tuple(wa.row_shape), dtype=torch.bfloat16, device="cuda", generator=g)
        v.view(total, -1).view(torch.int64)[:, 0] = torch.arange(total, device="cuda")   # row stamps
        return v

    x = rows_for(W.BASE_SEED + wa.index)
    a, b = torch.empty_like(x), torch.empty_like(x)
    rb = wa.row_bytes
    shifted = torch.empty((J, total), dtype=torch.int64, device="cuda")
    mask = torch.empty((J + 1, total), dtype=torch.uint8, device="cuda")
    status = torch.empty(1, dtype=torch.int32, device="cuda")

    def step(stream):
        thd.thd_build_route(route.handle, cu, n_slots, cp, total, stream)
        for _ in range(wa.layers):
            thd.thd_swap(route.handle, thd.Z2C, x, a, total, rb, stream)
            thd.thd_swap(route.handle, thd.C2Z, a, b, total, rb, stream)
        thd.thd_roll_labels_zigzag(route.handle, ids, cu, cu_real, n_slots, total, J, 0, shifted, mask, status,
                                   stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s.cuda_stream)                          # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    def check(w):
        assert route.status() == 0 and int(status.item()) == 0
        xh = x.view(total, -1).view(torch.int16).cpu().numpy()
        want_a = O.swap_rows(xh, w.cu_padded, cp, total, "z2c")
        assert np.array_equal(a.view(total, -1).view(torch.int16).cpu().numpy(), want_a)
        assert torch.equal(b.view(torch.int16), x.view(torch.int16))
        ws_, wm_ = O.roll_labels(w.ids(), w.cu_padded, w.cu_real, total, J, 0)
        for k in range(J):
            assert np.array_equal(shifted[k].cpu().numpy(), O.swap_rows(ws_[k], w.cu_padded, cp, total, "c2z"))
        for k in range(J + 1):
            assert np.array_equal(mask[k].cpu().numpy(), O.swap_rows(wm_[k], w.cu_padded, cp, total, "c2z"))

    for rep in range(2):
        a.zero_(); b.zero_(); shifted.fill_(-1); mask.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("full micro-batch graph replay", rep)
        check(wa)
        _ = (x.view(torch.int16)[:1024].float().sum() + 1).item()   # eager work between replays
    cu.copy_(dev_i32(wb.cu_padded))
    cu_real.copy_(dev_i32(wb.cu_real))
    x.copy_(rows_for(W.BASE_SEED + 77))
    ids.copy_(dev_i64(wb.ids()))
    a.zero_(); b.zero_(); shifted.fill_(-1); mask.fill_(7)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    say("full micro-batch graph replay with new boundaries")
    check(wb)


def test_graph_capture_of_the_whole_chain_from_token_rows(thd):
    # Pack -> route build -> zigzag roll -> multi-key swap captured in one
    # HIP graph (every shape fixed on the host by the token budget); replays
    # with eager work in between must match the oracle, and so must a replay
    # after new token rows are written into the captured input.
    import torch
    cp, batch, seq, max_docs = 4, 6, 1500, 120
    align = 2 * cp * 2
    capacity = ((batch * seq) // align + max_docs + 1) * align
    n_slots = max_docs + 1
    rows_a = W.token_rows(600, batch, seq, 0, 1, 0.004, 300, 0.0)
    rows_b = W.token_rows(601, batch, seq, 0, 1, 0.01, 100, 0.0)
    tokens = dev_i64(rows_a)
    nbytes = thd.thd_pack_workspace_bytes(batch, seq)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    packed = torch.empty(capacity, dtype=torch.int64, device="cuda")
    cu_real = torch.empty(max_docs + 2, dtype=torch.int32, device="cuda")
    cu_pad = torch.empty(max_docs + 2, dtype=torch.int32, device="cuda")
    pstatus = torch.empty(1, dtype=torch.int32, device="cuda")
    rstatus = torch.empty(1, dtype=torch.int32, device="cuda")
    route = thd.Route(n_slots, cp, capacity)
    shifted = torch.empty((2, capacity), dtype=torch.int64, device="cuda")
    mask = torch.empty((3, capacity), dtype=torch.uint8, device="cuda")
    pos = torch.arange(capacity, dtype=torch.int64, device="cuda")
    zig_tokens, zig_pos = torch.empty_like(packed), torch.empty_like(pos)

    def step(stream):
        thd.thd_pack(tokens, batch, seq, 0, 1, align, capacity, max_docs, 0, ws, nbytes, packed, cu_real, cu_pad,
                     pstatus, stream)
        thd.thd_build_route(route.handle, cu_pad, n_slots, cp, capacity, stream)
        thd.thd_roll_labels_zigzag(route.handle, packed, cu_pad, cu_real, n_slots, capacity, 2, -1, shifted, mask,
                                   rstatus, stream)
        thd.thd_swap_batch(route.handle, thd.C2Z, [packed, pos], [zig_tokens, zig_pos], [8, 8], capacity, stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    def check(rows):
        p, cr, cpd = O.pack_batch(rows, 0, 1, align, capacity, max_docs, 0)
        assert int(pstatus.item()) == 0 and int(rstatus.item()) == 0 and route.status() == 0
        assert np.array_equal(packed.cpu().numpy(), p)
        assert np.array_equal(cu_pad.cpu().numpy(), cpd) and np.array_equal(cu_real.cpu().numpy(), cr)
        ws_, wm_ = O.roll_labels(p, cpd, cr, capacity, 2, -1)
        for k in range(2):
            assert np.array_equal(shifted[k].cpu().numpy(), O.swap_rows(ws_[k], cpd, cp, capacity, "c2z"))
        for k in range(3):
            assert np.array_equal(mask[k].cpu().numpy(), O.swap_rows(wm_[k], cpd, cp, capacity, "c2z"))
        assert np.array_equal(zig_tokens.cpu().numpy(), O.swap_rows(p, cpd, cp, capacity, "c2z"))
        assert np.array_equal(zig_pos.cpu().numpy(), O.layout_tokens(cpd, cp, capacity, O.ZIGZAG))

    for rep in range(3):
        for t in (packed, shifted, zig_tokens, zig_pos):
            t.fill_(-3)
        mask.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("chain graph replay", rep)
        check(rows_a)
        _ = (pos.float().sum() + 1).item()           # eager work between replays
    tokens.copy_(dev_i64(rows_b))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    check(rows_b)
