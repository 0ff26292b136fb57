"""Error handling, identity, reuse and the no-host-wait property on the GPU.

Data errors are detected on the device and reported through the status word;
a swap on a route with a bad status, and a roll with bad boundaries, write
nothing (their outputs keep a sentinel).  Host-detectable misuse returns its
code at once.  None of these cases makes a kernel fault: bad boundaries are
read but never used as addresses.
"""

import time

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import CODE_OF_KIND, check_route_matches_oracle, dev_i32, dev_i64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def thd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_packed_sequence_amd as thd
    return thd


BAD_ROUTES = [
    ([0, 6, 16], 2, 16),
    ([1, 8, 16], 2, 16),
    ([0, 8, 4, 16], 2, 16),
    ([0, 8, 16], 2, 24),
    ([2, 1, 7], 2, 9),
    ([0, 9, 3, 12], 2, 16),
    ([0, 6, 12], 2, 16),
    ([0, 8, 16, 8], 4, 8),
    ([0, -8, 8], 2, 8),
]


@pytest.mark.parametrize("cu,cp,total", BAD_ROUTES)
def test_bad_boundaries_give_the_oracle_kind_and_write_nothing(thd, cu, cp, total):
    import torch
    with pytest.raises(O.OracleInputError) as e:
        O.build_route(cu, cp, total)
    want = CODE_OF_KIND[e.value.kind]
    say("bad route", cu, cp, total, e.value.kind)
    route = thd.Route(len(cu) - 1, cp, total)
    route.build(dev_i32(cu), cp, total)
    assert route.status() == want
    x = torch.arange(total * 4, dtype=torch.int32, device="cuda").view(total, 4)
    out = torch.full_like(x, -77)
    code = thd.thd_swap(route.handle, thd.Z2C, x, out, total, 16)
    assert code == thd.THD_OK             # the launch happens; the kernel sees the status and stops
    torch.cuda.synchronize()
    assert (out == -77).all()
    by_src, _, _ = route.copy_out()
    assert by_src.shape[0] == 0


def test_rebuild_after_error_recovers(thd):
    import torch
    route = thd.Route(4, 2, 16)
    route.build(dev_i32([0, 6, 16]), 2, 16)
    assert route.status() == thd.THD_ERR_CU_DIVISIBLE
    route.build(dev_i32([0, 4, 8, 16]), 2, 16)
    check_route_matches_oracle(route, [0, 4, 8, 16], 2, 16)


ROLL_ERRORS = [
    ([1, 4, 8], [0, 3, 6], 8),
    ([0, 4, 8], [1, 3, 6], 8),
    ([0, 4, 2, 8], [0, 3, 3, 6], 8),
    ([0, 4, 8], [0, 3, 2], 8),
    ([0, 4, 8], [0, 3, 6], 12),
    ([0, 4, 8], [0, 5, 6], 8),
]


@pytest.mark.parametrize("cu_pad,cu_real,total", ROLL_ERRORS)
def test_roll_errors(thd, cu_pad, cu_real, total):
    import torch
    with pytest.raises(O.OracleInputError) as e:
        O.roll_labels(np.zeros(total, np.int64), cu_pad, cu_real, total, 2)
    say("bad roll", cu_pad, cu_real, total, e.value.kind)
    ids = torch.arange(total, dtype=torch.int64, device="cuda")
    shifted = torch.full((2, total), -3, dtype=torch.int64, device="cuda")
    mask = torch.full((3, total), 9, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), 123, dtype=torch.int32, device="cuda")
    code = thd.thd_roll_labels(ids, dev_i32(cu_pad), dev_i32(cu_real), len(cu_pad) - 1, total, 2, 0,
                               shifted, mask, status)
    assert code == thd.THD_OK
    torch.cuda.synchronize()
    assert int(status.item()) == CODE_OF_KIND[e.value.kind]
    assert (shifted == -3).all() and (mask == 9).all()


def test_host_side_errors(thd):
    import torch
    route = thd.Route(8, 4, 64)
    x = torch.zeros(32, 8, dtype=torch.uint8, device="cuda")
    y = torch.zeros_like(x)
    with pytest.raises(thd.ThdError) as e:
        thd.thd_swap(route.handle, thd.Z2C, x, y, 32, 8)
    assert e.value.code == thd.THD_ERR_NOT_BUILT
    route.build(dev_i32([0, 16, 32]), 2, 32)
    for args, code in [
        ((route.handle, 2, x, y, 32, 8), thd.THD_ERR_DIRECTION),
        ((route.handle, -1, x, y, 32, 8), thd.THD_ERR_DIRECTION),
        ((route.handle, thd.Z2C, x, y, 16, 8), thd.THD_ERR_SHAPE),
        ((route.handle, thd.Z2C, x, x, 32, 8), thd.THD_ERR_ALIAS),
        ((route.handle, thd.Z2C, x.data_ptr(), x.data_ptr() + 8, 32, 8), thd.THD_ERR_ALIAS),
        ((route.handle, thd.Z2C, x, y, 32, 0), thd.THD_ERR_ARG),
        ((route.handle, thd.Z2C, 0, y, 32, 8), thd.THD_ERR_ARG),
    ]:
        with pytest.raises(thd.ThdError) as e:
            thd.thd_swap(*args)
        assert e.value.code == code, args
    cu = dev_i32([0, 16, 32])
    for args, code in [
        ((route.handle, cu, 2, 8, 32), thd.THD_ERR_CAPACITY),      # cp above max_cp
        ((route.handle, cu, 9, 2, 32), thd.THD_ERR_CAPACITY),      # n_slots above max_slots
        ((route.handle, cu, 2, 2, 65), thd.THD_ERR_CAPACITY),      # tokens above max_tokens
        ((route.handle, cu, -1, 2, 32), thd.THD_ERR_ARG),
        ((route.handle, cu, 2, 0, 32), thd.THD_ERR_ARG),
    ]:
        with pytest.raises(thd.ThdError) as e:
            thd.thd_build_route(*args)
        assert e.value.code == code, args
    # a rejected build leaves the last good route usable
    out = route.swap(x, thd.Z2C)
    torch.cuda.synchronize()
    assert out.shape == x.shape
    # the wrappers refuse output buffers that do not match the input before
    # any launch (the C ABI would write rows x row_bytes bytes into them)
    short = torch.zeros(31, 8, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="elements"):
        route.swap(x, thd.Z2C, out=short)
    with pytest.raises(ValueError, match="must be torch.uint8"):
        route.swap(x, thd.Z2C, out=torch.zeros(32, 8, dtype=torch.int16, device="cuda"))
    with pytest.raises(ValueError, match="rows"):
        route.swap_many([x, torch.zeros(16, 8, dtype=torch.uint8, device="cuda")], thd.Z2C)
    with pytest.raises(ValueError, match="elements"):
        route.swap_many([x], thd.Z2C, outs=[short])
    assert (short == 0).all()


def test_identity_routes(thd):
    import torch
    route = thd.Route(4, 4, 64)
    x = torch.arange(64, dtype=torch.int64, device="cuda").view(16, 4)
    route.build(dev_i32([0, 3, 16]), 1, 16)         # cp == 1: the boundaries are not even checked
    assert route.swap(x, thd.Z2C) is x and route.swap(x, thd.C2Z) is x
    assert thd.thd_swap(route.handle, thd.Z2C, x, torch.empty_like(x), 16, 32) == thd.THD_IDENTITY
    assert route.status() == 0
    route.build(dev_i32([0, 0, 0]), 2, 0)            # empty batch
    assert route.status() == 0
    # an empty batch of many slots (enough segments for the closed-form
    # build, which needs a document): zero runs, zero split, status OK
    many = thd.Route(600, 8, 64)
    many.build(dev_i32([0] * 601), 8, 0)
    check_route_matches_oracle(many, np.zeros(601, dtype=np.int64), 8, 0)
    many.close()
    empty = torch.empty(0, 4, dtype=torch.int64, device="cuda")
    assert thd.thd_swap(route.handle, thd.Z2C, empty, torch.empty_like(empty), 0, 32) == thd.THD_IDENTITY
    shifted, mask, status = thd.roll_labels(torch.empty(0, dtype=torch.int64, device="cuda"), dev_i32([0]), None, 2)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and shifted.numel() == 0


def test_route_reuse_and_rebuild(thd):
    # One route serves many swaps; rebuilding for new boundaries or a new cp
    # gives the new route (Relax PR #273 §5: rebuild on new boundaries, on a cp change).
    import torch
    route = thd.Route(64, 8, 4096)
    cases = [(W.random_packed(s, cp, 12, 20, 2, row_shape=(16,), row_dtype="uint8"), cp)
             for s, cp in ((1, 2), (2, 4), (3, 8), (4, 4))]
    for w, cp in cases:
        if w.total > 4096 or w.n_slots > 64:
            continue
        say("reuse", w.name, cp, w.total)
        route.build(dev_i32(w.cu_padded), cp, w.total)
        x = torch.from_numpy(w.rows_host()).cuda()
        cur = x
        for _ in range(10):
            cur = route.swap(route.swap(cur, thd.Z2C), thd.C2Z)
        z = route.swap(cur, thd.Z2C)
        torch.cuda.synchronize()
        assert torch.equal(cur, x)
        assert np.array_equal(z.cpu().numpy(), O.swap_rows(w.rows_host(), w.cu_padded, cp, w.total, "z2c"))
        check_route_matches_oracle(route, w.cu_padded, cp, w.total)


def test_calls_never_wait_for_the_gpu(thd):
    # Hold the stream with a long spin kernel, then enqueue the whole hot path
    # of one micro-batch (build, 96 swaps, roll).  If any call synchronised,
    # it could only return after the spin ended; the spin must still be running
    # when the last call has returned.
    import torch
    w = W.make("full")
    total, cp = w.total, w.cp
    route = thd.Route(w.n_slots, cp, total)
    cu = dev_i32(w.cu_padded)
    cu_real = dev_i32(w.cu_real)
    ids = dev_i64(w.ids())
    x = torch.randn(total, 2048, dtype=torch.bfloat16, device="cuda")
    a, b = torch.empty_like(x), torch.empty_like(x)
    shifted = torch.empty((w.max_shift, total), dtype=torch.int64, device="cuda")
    mask = torch.empty((w.max_shift + 1, total), dtype=torch.uint8, device="cuda")
    status = torch.empty(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    say("gate: spin then enqueue")
    start, gate_done = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    torch.cuda._sleep(int(5e8))
    gate_done.record()
    t0 = time.perf_counter()
    route.build(cu, cp, total)
    for _ in range(w.layers):
        route.swap(x, thd.Z2C, out=a)
        route.swap(a, thd.C2Z, out=b)
    thd.thd_roll_labels(ids, cu, cu_real, w.n_slots, total, w.max_shift, 0, shifted, mask, status)
    enqueue_s = time.perf_counter() - t0
    still_spinning = not gate_done.query()
    torch.cuda.synchronize()
    gate_ms = start.elapsed_time(gate_done)
    say(f"enqueue {enqueue_s * 1e3:.2f} ms, gate {gate_ms:.1f} ms, still spinning {still_spinning}")
    assert still_spinning, "a call waited for the GPU"
    assert gate_ms > enqueue_s * 1e3
    assert torch.equal(b, x)
    assert int(status.item()) == 0


def test_side_streams_and_two_routes(thd):
    # Two routes built and used on two non-default streams, interleaved; each
    # stream's work is ordered, the routes share nothing.
    import torch
    wa = W.random_packed(900, 4, 40, 30, 3, row_shape=(64,), row_dtype="uint8")
    wb = W.random_packed(901, 8, 25, 20, 5, row_shape=(64,), row_dtype="uint8")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ra = thd.Route(wa.n_slots, wa.cp, wa.total)
    rb = thd.Route(wb.n_slots, wb.cp, wb.total)
    xa = torch.from_numpy(wa.rows_host()).cuda()
    xb = torch.from_numpy(wb.rows_host()).cuda()
    cua, cub = dev_i32(wa.cu_padded), dev_i32(wb.cu_padded)
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        ra.build(cua, wa.cp, wa.total, stream=sa.cuda_stream)
        ya = ra.swap(xa, thd.Z2C, stream=sa.cuda_stream)
    with torch.cuda.stream(sb):
        rb.build(cub, wb.cp, wb.total, stream=sb.cuda_stream)
        yb = rb.swap(xb, thd.C2Z, stream=sb.cuda_stream)
    with torch.cuda.stream(sa):
        za = ra.swap(ya, thd.C2Z, stream=sa.cuda_stream)
    torch.cuda.synchronize()
    assert ra.status(sa.cuda_stream) == 0 and rb.status(sb.cuda_stream) == 0
    assert np.array_equal(ya.cpu().numpy(), O.swap_rows(wa.rows_host(), wa.cu_padded, wa.cp, wa.total, "z2c"))
    assert np.array_equal(yb.cpu().numpy(), O.swap_rows(wb.rows_host(), wb.cu_padded, wb.cp, wb.total, "c2z"))
    assert torch.equal(za, xa)
