"""The five named workloads at full size, in the launch configuration the bench
times (default swap tiles, one workgroup per tile, non-temporal streaming).

* the route (runs in both orders, split matrix) equals the oracle's exactly;
* every output row's origin is checked through a stamp: each input row's
  first 8 bytes hold its row index, so the stamps read back from the output
  must equal the oracle's source row for every output row;
* sampled rows (random ones plus the first and last row of every run) are
  compared byte for byte with the input row the oracle names;
* every output byte is compared with the input row the oracle names for
  it: the oracle's source-row list gathers the input on the device, 256 MiB
  of output at a time, and the two must be equal (all workloads, the 16 GiB
  long1m swaps included);
* z->c followed by c->z returns the input exactly; where the buffers fit
  comfortably in host memory the whole output is also compared with the
  oracle's swap computed on the host.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import check_route_matches_oracle, dev_i32, dev_i64, oracle_source_rows, say

pytestmark = pytest.mark.gpu

FULL_COMPARE = {"tiny", "gdn128k", "sft", "full"}


@pytest.fixture(scope="module")
def thd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_packed_sequence_amd as thd
    return thd


def device_rows(w):
    import torch
    g = torch.Generator(device="cuda").manual_seed(W.BASE_SEED + w.index)
    x = torch.randn((w.total,) + tuple(w.row_shape), dtype=torch.bfloat16, device="cuda", generator=g)
    x.view(w.total, -1).view(torch.int64)[:, 0] = torch.arange(w.total, device="cuda")
    return x


def assert_every_row_from_oracle_source(out, x, src, chunk_bytes=256 << 20):
    """out[j] == x[src[j]] for every row j, byte for byte: the oracle's
    source-row list gathers the expected rows on the device, chunk by chunk."""
    import torch
    total = out.shape[0]
    o = out.view(total, -1).view(torch.uint8)
    xi = x.view(total, -1).view(torch.uint8)
    rows = max(1, chunk_bytes // o.shape[1])
    src_t = torch.from_numpy(np.ascontiguousarray(src, dtype=np.int64)).cuda()
    for a in range(0, total, rows):
        b = min(total, a + rows)
        want = xi.index_select(0, src_t[a:b])
        assert torch.equal(o[a:b], want), f"rows {a}..{b}"
        del want


def sample_rows(runs, total, rng, n=4096):
    idx = rng.integers(0, total, size=min(n, total))
    edges = np.concatenate([runs[:, 1], runs[:, 1] + runs[:, 2] - 1, runs[:, 0], runs[:, 0] + runs[:, 2] - 1])
    return np.unique(np.concatenate([idx, edges, [0, total - 1]]))


@pytest.mark.parametrize("name", list(W.NAMES) + ["sft512"])
def test_workload_parity(thd, name):
    import torch
    w = W.make(name)
    total, cp = w.total, w.cp
    say("workload", name, "T", total, "cp", cp, "slots", w.n_slots, "row_bytes", w.row_bytes)
    route = thd.Route(w.n_slots, cp, total)
    route.build(dev_i32(w.cu_padded), cp, total)
    r = check_route_matches_oracle(route, w.cu_padded, cp, total)
    runs = O.canonical_runs(r)
    x = device_rows(w)
    rng = np.random.default_rng(5)
    for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
        say(" swap", name, direction)
        out = route.swap(x, d)
        torch.cuda.synchronize()
        src = oracle_source_rows(r, direction)
        stamps = out.view(total, -1).view(torch.int64)[:, 0].cpu().numpy()
        assert np.array_equal(stamps, src)
        rows = sample_rows(runs, total, rng)
        rows_t = torch.from_numpy(rows).cuda()
        got = out.view(total, -1).index_select(0, rows_t).view(torch.int16).cpu().numpy()
        want = x.view(total, -1).index_select(0, torch.from_numpy(src[rows]).cuda()).view(torch.int16).cpu().numpy()
        assert np.array_equal(got, want)
        assert_every_row_from_oracle_source(out, x, src)
        back = route.swap(out, thd.C2Z if d == thd.Z2C else thd.Z2C)
        torch.cuda.synchronize()
        assert torch.equal(back.view(torch.int16), x.view(torch.int16))
        if name in FULL_COMPARE:
            xh = x.view(total, -1).view(torch.int16).cpu().numpy()
            want_all = O.swap_rows(xh, w.cu_padded, cp, total, direction)
            assert np.array_equal(out.view(total, -1).view(torch.int16).cpu().numpy(), want_all)
        del out, back
    del x
    torch.cuda.empty_cache()


def test_full_microbatch_96_swaps_and_roll(thd):
    # One route reused by 48 layers x (z->c, c->z), then the label/MTP roll.
    import torch
    w = W.make("full")
    total, cp = w.total, w.cp
    say("full micro-batch", total, cp)
    route = thd.Route(w.n_slots, cp, total)
    route.build(dev_i32(w.cu_padded), cp, total)
    x = device_rows(w)
    a = torch.empty_like(x)
    b = torch.empty_like(x)
    cur = x
    for layer in range(w.layers):
        route.swap(cur, thd.Z2C, out=a)
        route.swap(a, thd.C2Z, out=b)
        cur = b
    torch.cuda.synchronize()
    assert torch.equal(b.view(torch.int16), x.view(torch.int16))
    r = O.build_route(w.cu_padded.tolist(), cp, total)
    stamps = a.view(total, -1).view(torch.int64)[:, 0].cpu().numpy()
    assert np.array_equal(stamps, oracle_source_rows(r, "z2c"))
    ids = w.ids()
    shifted, mask, status = thd.roll_labels(dev_i64(ids), dev_i32(w.cu_padded), dev_i32(w.cu_real), w.max_shift, 0)
    torch.cuda.synchronize()
    want_s, want_m = O.roll_labels(ids, w.cu_padded, w.cu_real, total, w.max_shift, 0)
    assert int(status.item()) == 0
    assert np.array_equal(shifted.cpu().numpy(), want_s)
    assert np.array_equal(mask.cpu().numpy(), want_m)
    # valid-token count identity: sum of the mask equals the sum of real lengths
    assert int(mask[0].sum().item()) == int(np.diff(w.cu_real).sum())


@pytest.mark.parametrize("name", ["tiny", "gdn128k", "sft"])
def test_workload_roll(thd, name):
    import torch
    w = W.make(name)
    ids = w.ids()
    say("roll workload", name)
    shifted, mask, status = thd.roll_labels(dev_i64(ids), dev_i32(w.cu_padded), dev_i32(w.cu_real), 4, -1)
    torch.cuda.synchronize()
    want_s, want_m = O.roll_labels(ids, w.cu_padded, w.cu_real, w.total, 4, -1)
    assert int(status.item()) == 0
    assert np.array_equal(shifted.cpu().numpy(), want_s)
    assert np.array_equal(mask.cpu().numpy(), want_m)


def test_maximum_size_swap(thd):
    # T = 2**31 - 64 tokens (int32 boundaries at their limit), 1-byte rows:
    # 2 GiB per buffer.  The route is checked run by run and token by token
    # with the oracle's single-token form; the swap on sampled rows and by the
    # round trip.
    import torch
    cp = 2
    total = 2 ** 31 - 64
    lens = [1 << 29, 123456788, 4, 1000000000, 0]
    lens[-1] = total - sum(lens[:-1])
    assert all(v % (2 * cp) == 0 for v in lens) and sum(lens) == total
    cu = W.cumulative(lens)
    say("maximum size", total)
    route = thd.Route(len(lens), cp, total)
    route.build(dev_i32(cu), cp, total)
    assert route.status() == 0
    by_src, by_dst, split = route.copy_out()
    share = total // cp
    assert (split.astype(np.int64).sum(0) == share).all() and (split.astype(np.int64).sum(1) == share).all()
    for order, col in ((by_src, 0), (by_dst, 1)):
        starts = order[:, col].astype(np.int64)
        assert starts[0] == 0 and np.array_equal(starts[1:], starts[:-1] + order[:-1, 2])
        assert int(order[:, 2].astype(np.int64).sum()) == total
    for zrow, tok, n in by_src.astype(np.int64):
        for off in (0, n - 1):
            assert O.zigzag_position(cu, cp, total, int(tok + off)) == zrow + off
    x = torch.randint(0, 256, (total, 1), dtype=torch.uint8, device="cuda")
    out = route.swap(x, thd.Z2C)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([rng.integers(0, total, 3000), by_src[:, 1].astype(np.int64),
                                     by_src[:, 1].astype(np.int64) + by_src[:, 2] - 1, [0, total - 1]]))
    src = np.array([O.zigzag_position(cu, cp, total, int(t)) for t in toks], dtype=np.int64)
    got = out.view(-1).index_select(0, torch.from_numpy(toks).cuda()).cpu().numpy()
    want = x.view(-1).index_select(0, torch.from_numpy(src).cuda()).cpu().numpy()
    assert np.array_equal(got, want)
    back = route.swap(out, thd.C2Z)
    torch.cuda.synchronize()
    assert torch.equal(back, x)
    del x, out, back, route
    torch.cuda.empty_cache()


def _many_documents(total, n, align, seed):
    rng = np.random.default_rng([W.BASE_SEED, seed])
    raw = rng.integers(1, 1000, n).astype(np.float64)
    lens = (np.floor(raw / raw.sum() * total / align) * align).astype(np.int64)
    lens = np.maximum(lens, align)  # no empty document
    lens[-1] += total - lens.sum()
    assert (lens % align == 0).all() and lens.sum() == total and (lens > 0).all()
    return W.cumulative(lens)


@pytest.mark.parametrize("log2_total,n_docs", [(24, 40), (24, 520), (19, 130)])
def test_route_build_above_the_workgroup_cap(thd, log2_total, n_docs):
    # cp 8.  T = 2**24 (2**20 directory blocks) over 40 documents (640 zigzag
    # segments): the one-launch build, whose grid is capped below the blocks
    # it would need at 1024 per workgroup, so each workgroup writes a larger
    # share; over 520 documents (8320 segments): the closed-form runs, whose
    # workgroups would hold over 2048 directory entries each, then the
    # directory launch.  T = 2**19 over 130 documents (2080 segments, 17
    # workgroups of 128): the closed-form runs writing about 1900 directory
    # entries per workgroup in the same launch, two passes of the threads.
    # 16-byte rows with 16-byte tiles make every row its own tile, so every
    # directory entry is read by the swap; every output row is then compared
    # with the input row the oracle's zigzag layout names for it (c->z: row i
    # holds token zigzag[i]; z->c: token g comes from the row holding it).
    import torch
    cp, total = 8, 1 << log2_total
    cu = _many_documents(total, n_docs, 2 * cp, 78)
    say("route above the workgroup cap: T", total, "slots", len(cu) - 1)
    route = thd.Route(len(cu) - 1, cp, total)
    route.build(dev_i32(cu), cp, total)
    assert route.status() == 0
    zig = O.layout_tokens(cu, cp, total, O.ZIGZAG)
    row_of = np.empty_like(zig)
    row_of[zig] = np.arange(total, dtype=zig.dtype)
    g = torch.Generator(device="cuda").manual_seed(W.BASE_SEED + 79)
    x = torch.empty((total, 16), dtype=torch.uint8, device="cuda")
    x.view(torch.int64).random_(generator=g)
    thd.thd_route_launch_shape(route.handle, 16, 1, 0, 0)
    for direction, d, src in (("z2c", thd.Z2C, row_of), ("c2z", thd.C2Z, zig)):
        out = route.swap(x, d)
        torch.cuda.synchronize()
        assert_every_row_from_oracle_source(out, x, src)
        del out
    del x
    torch.cuda.empty_cache()


def test_maximum_size_route_with_many_documents(thd):
    # T = 2**31 - 64 tokens over 520 documents at cp 8: the build (runs in
    # closed form, then the directory launch) stays within a few
    # milliseconds, every run
    # starts and ends where the oracle's single-token form puts its tokens,
    # and a 1-byte-row swap matches that form on sampled tokens and returns
    # the input on the round trip.
    import torch
    cp, total = 8, 2 ** 31 - 64
    cu = _many_documents(total, 520, 2 * cp, 80)
    say("maximum size, many documents: T", total, "slots", len(cu) - 1)
    route = thd.Route(len(cu) - 1, cp, total)
    cu_d = dev_i32(cu)
    route.build(cu_d, cp, total)
    torch.cuda.synchronize()
    times = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        route.build(cu_d, cp, total)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    say("build ms", [round(t, 3) for t in times])
    assert float(np.median(times)) < 5.0
    assert route.status() == 0
    by_src, by_dst, split = route.copy_out()
    share = total // cp
    assert (split.astype(np.int64).sum(0) == share).all() and (split.astype(np.int64).sum(1) == share).all()
    for order, col in ((by_src, 0), (by_dst, 1)):
        starts = order[:, col].astype(np.int64)
        assert starts[0] == 0 and np.array_equal(starts[1:], starts[:-1] + order[:-1, 2])
    for zrow, tok, n in by_src.astype(np.int64):
        for off in (0, n - 1):
            assert O.zigzag_position(cu, cp, total, int(tok + off)) == zrow + off
    x = torch.randint(0, 256, (total, 1), dtype=torch.uint8, device="cuda")
    out = route.swap(x, thd.Z2C)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    toks = np.unique(np.concatenate([rng.integers(0, total, 3000), by_src[:, 1].astype(np.int64),
                                     by_src[:, 1].astype(np.int64) + by_src[:, 2] - 1, [0, total - 1]]))
    src = np.array([O.zigzag_position(cu, cp, total, int(t)) for t in toks], dtype=np.int64)
    got = out.view(-1).index_select(0, torch.from_numpy(toks).cuda()).cpu().numpy()
    want = x.view(-1).index_select(0, torch.from_numpy(src).cuda()).cpu().numpy()
    assert np.array_equal(got, want)
    back = route.swap(out, thd.C2Z)
    torch.cuda.synchronize()
    assert torch.equal(back, x)
    del x, out, back, route
    torch.cuda.empty_cache()


def test_maximum_size_swap_wide_rows(thd):
    # T = 2**31 - 64 tokens of 16-byte rows (the widest copy unit): 32 GiB
    # per buffer, so every byte offset past 2**31 and 2**32 is exercised on
    # the 4 KiB-tile path.  Sampled rows against the oracle's single-token
    # form, every run's first and last token included; then the round trip.
    import torch
    cp = 4
    total = 2 ** 31 - 64
    lens = [1 << 30, 8, 0, 536870912, 24, total - (1 << 30) - 536870912 - 32]
    assert all(v % (2 * cp) == 0 for v in lens) and sum(lens) == total
    cu = W.cumulative(lens)
    say("maximum size, 16-byte rows", total)
    route = thd.Route(len(lens), cp, total)
    route.build(dev_i32(cu), cp, total)
    assert route.status() == 0
    by_src, _, _ = route.copy_out()
    g = torch.Generator(device="cuda").manual_seed(W.BASE_SEED + 41)
    x = torch.empty((total, 16), dtype=torch.uint8, device="cuda")
    x.view(torch.int64).random_(generator=g)
    out = route.swap(x, thd.Z2C)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([rng.integers(0, total, 3000), by_src[:, 1].astype(np.int64),
                                     by_src[:, 1].astype(np.int64) + by_src[:, 2] - 1, [0, total - 1]]))
    src = np.array([O.zigzag_position(cu, cp, total, int(t)) for t in toks], dtype=np.int64)
    got = out.index_select(0, torch.from_numpy(toks).cuda()).cpu().numpy()
    want = x.index_select(0, torch.from_numpy(src).cuda()).cpu().numpy()
    assert np.array_equal(got, want)
    back = route.swap(out, thd.C2Z)
    torch.cuda.synchronize()
    assert torch.equal(back, x)
    del x, out, back, route
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rb", [3, 12])
def test_maximum_size_swap_narrow_rows(thd, rb):
    # T = 2**31 - 64 tokens of 3- and 12-byte rows (1- and 4-byte copy units,
    # run pieces realigned onto 16-byte stores): 6 and 24 GiB per buffer, so
    # the realigning copy runs at byte offsets past 2**32.  Sampled rows
    # against the oracle's single-token form, every run's first and last
    # token included; then the round trip.
    import torch
    cp = 4
    total = 2 ** 31 - 64
    lens = [8, 1 << 30, 16, 536870912, 24, total - (1 << 30) - 536870912 - 48]
    assert all(v % (2 * cp) == 0 for v in lens) and sum(lens) == total
    cu = W.cumulative(lens)
    say("maximum size, narrow rows", rb, total)
    route = thd.Route(len(lens), cp, total)
    route.build(dev_i32(cu), cp, total)
    assert route.status() == 0
    by_src, _, _ = route.copy_out()
    g = torch.Generator(device="cuda").manual_seed(W.BASE_SEED + 43 + rb)
    x = torch.empty((total, rb), dtype=torch.uint8, device="cuda")
    if rb % 4 == 0:
        x.view(torch.int32).random_(generator=g)
    else:
        x.random_(0, 256, generator=g)
    out = route.swap(x, thd.Z2C)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7 + rb)
    toks = np.unique(np.concatenate([rng.integers(0, total, 3000), by_src[:, 1].astype(np.int64),
                                     by_src[:, 1].astype(np.int64) + by_src[:, 2] - 1, [0, total - 1]]))
    src = np.array([O.zigzag_position(cu, cp, total, int(t)) for t in toks], dtype=np.int64)
    got = out.index_select(0, torch.from_numpy(toks).cuda()).cpu().numpy()
    want = x.index_select(0, torch.from_numpy(src).cuda()).cpu().numpy()
    assert np.array_equal(got, want)
    back = route.swap(out, thd.C2Z)
    torch.cuda.synchronize()
    assert torch.equal(back, x)
    del x, out, back, route
    torch.cuda.empty_cache()


def test_maximum_size_swap_batch(thd):
    # T = 2**31 - 64 tokens through the multi-tensor swap in one launch: a
    # uint8 key, 3-byte rows and an int64 key (2, 6 and 16 GiB per buffer).
    # Sampled rows against the oracle's single-token form, every run's first
    # and last token included; then the round trip.
    import torch
    cp = 4
    total = 2 ** 31 - 64
    lens = [16, 1 << 30, 8, 536870912, 24, total - (1 << 30) - 536870912 - 48]
    assert all(v % (2 * cp) == 0 for v in lens) and sum(lens) == total
    cu = W.cumulative(lens)
    say("maximum size, multi-tensor swap", total)
    route = thd.Route(len(lens), cp, total)
    route.build(dev_i32(cu), cp, total)
    assert route.status() == 0
    by_src, _, _ = route.copy_out()
    g = torch.Generator(device="cuda").manual_seed(W.BASE_SEED + 47)
    xs = [torch.empty((total, 1), dtype=torch.uint8, device="cuda"),
          torch.empty((total, 3), dtype=torch.uint8, device="cuda"),
          torch.empty((total,), dtype=torch.int64, device="cuda")]
    xs[0].random_(0, 256, generator=g)
    xs[1].random_(0, 256, generator=g)
    xs[2].random_(generator=g)
    outs = route.swap_many(xs, thd.Z2C)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    toks = np.unique(np.concatenate([rng.integers(0, total, 3000), by_src[:, 1].astype(np.int64),
                                     by_src[:, 1].astype(np.int64) + by_src[:, 2] - 1, [0, total - 1]]))
    src = np.array([O.zigzag_position(cu, cp, total, int(t)) for t in toks], dtype=np.int64)
    t_toks, t_src = torch.from_numpy(toks).cuda(), torch.from_numpy(src).cuda()
    for i, (x, o) in enumerate(zip(xs, outs)):
        assert torch.equal(o.index_select(0, t_toks), x.index_select(0, t_src)), f"tensor {i}"
    backs = route.swap_many(outs, thd.C2Z)
    torch.cuda.synchronize()
    for i, (x, b) in enumerate(zip(xs, backs)):
        assert torch.equal(b, x), f"tensor {i}"
    del xs, outs, backs, route
    torch.cuda.empty_cache()


def test_maximum_size_roll(thd):
    # T = 2**31 - 64 positions, two shifts: the label and MTP outputs reach
    # 2 x 16 GiB, so every index past 2**31 is exercised.  Checked at sampled
    # positions (random ones and every position near a slot's real end and
    # padded end) with the oracle's single-position form, in natural order
    # and written in the zigzag order of a cp = 2 route.
    import torch
    cp, j_max, fill = 2, 2, -5
    total = 2 ** 31 - 64
    lens = [1 << 29, 123456788, 4, 1000000000, 0]
    lens[-1] = total - sum(lens[:-1])
    real = [lens[0] - 3, lens[1], 1, lens[3] - 2, lens[4] - 1]
    cu, cu_r = W.cumulative(lens), W.cumulative(real)
    say("maximum size roll", total)
    g = torch.Generator(device="cuda").manual_seed(W.BASE_SEED + 31)
    ids = torch.randint(0, 32000, (total,), dtype=torch.int64, device="cuda", generator=g)
    rng = np.random.default_rng(4)
    edges = []
    for s in range(len(lens)):
        e = int(cu[s]) + real[s]
        edges += [int(cu[s]), int(cu[s]) + 1, e - 3, e - 2, e - 1, e, int(cu[s + 1]) - 1]
    toks = np.unique(np.clip(np.concatenate([rng.integers(0, total, 3000), edges, [0, total - 1]]), 0, total - 1))
    toks_t = torch.from_numpy(toks).cuda()
    # ids the labels may read: t + j for every sampled t and shift
    ahead = {j: ids.index_select(0, torch.from_numpy(np.minimum(toks + j, total - 1)).cuda()).cpu().numpy()
             for j in range(1, j_max + 1)}
    valid = {j: np.array([O.roll_valid_at(cu, cu_r, int(t), j) for t in toks]) for j in range(j_max + 1)}

    def check(shifted, mask, rows):
        rows_t = torch.from_numpy(rows).cuda()
        for j in range(j_max + 1):
            assert np.array_equal(mask[j].index_select(0, rows_t).cpu().numpy(), valid[j].astype(np.uint8)), j
            if j:
                want = np.where(valid[j], ahead[j], fill)
                assert np.array_equal(shifted[j - 1].index_select(0, rows_t).cpu().numpy(), want), j

    shifted, mask, status = thd.roll_labels(ids, dev_i32(cu), dev_i32(cu_r), j_max, fill)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    check(shifted, mask, toks)
    assert int(mask[0].sum(dtype=torch.int64).item()) == sum(real)
    del shifted, mask
    torch.cuda.empty_cache()

    route = thd.Route(len(lens), cp, total)
    route.build(dev_i32(cu), cp, total)
    shifted, mask, status = route.roll_labels_zigzag(ids, dev_i32(cu), dev_i32(cu_r), j_max, fill)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    rows = np.array([O.zigzag_position(cu, cp, total, int(t)) for t in toks], dtype=np.int64)
    check(shifted, mask, rows)
    del shifted, mask, ids, route
    torch.cuda.empty_cache()
