"""GPU parity: libthdcp against the CPU oracle, byte for byte.

Everything here is integer index work and bit copies, so the bar is exact
equality: the route (runs in both orders and the split matrix), every swapped
byte, every label and every mask byte.  Cases are small enough for the oracle
to finish in seconds but span many swap tiles and end in a ragged tail.
"""

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import check_route_matches_oracle, dev_i32, dev_i64, expected_route, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def thd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_packed_sequence_amd as thd
    return thd


def build(thd, cu, cp, total, max_slots=None, max_cp=None):
    route = thd.Route(max_slots or max(1, len(cu) - 1), max_cp or cp, max(total, 1))
    route.build(dev_i32(cu), cp, total)
    return route


# ---- the test matrix of the Relax PR #273 page, §5: cp x direction x shape ----

SHAPES = {
    "single": [0, 48],
    "unequal": [0, 16, 64, 96, 208],
    "repeated": [0, 0, 32, 32, 32, 96, 160, 160],
}


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("direction", ["z2c", "c2z"])
@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_matrix_route_and_swap(thd, cp, direction, shape):
    import torch
    base = SHAPES[shape]
    unit = 2 * cp
    cu = [v // 16 * unit for v in base]          # same shape, lengths scaled to multiples of 2*cp
    total = cu[-1]
    say("matrix", cp, direction, shape, cu)
    route = build(thd, cu, cp, total)
    x = torch.randint(0, 256, (total, 24), dtype=torch.uint8, device="cuda")
    d = thd.Z2C if direction == "z2c" else thd.C2Z
    out = route.swap(x, d)
    torch.cuda.synchronize()
    if cp == 1:
        assert out is x
        return
    check_route_matches_oracle(route, cu, cp, total)
    want = O.swap_rows(x.cpu().numpy(), cu, cp, total, direction)
    assert np.array_equal(out.cpu().numpy(), want)
    # neighbouring ranks agree on split sizes: sender row s == receiver column s
    _, _, split = route.copy_out()
    r, _ = expected_route(cu, cp, total)
    for s in range(cp):
        assert split[s, :].tolist() == r["input_split_sizes"][s].tolist()
        assert split[:, s].tolist() == r["output_split_sizes"][s].tolist()


# ---- random ragged batches, many row sizes and alignments ----

RANDOM_CASES = [
    # seed, cp, docs, max_chunk, empty slots, row bytes, byte offset of both buffers
    (0, 2, 9, 40, 0, 32, 0),
    (1, 4, 40, 64, 3, 16, 0),
    (2, 8, 25, 20, 8, 4096, 0),
    (3, 3, 30, 50, 2, 12, 0),
    (4, 4, 33, 48, 1, 4, 4),
    (5, 2, 50, 70, 5, 6, 2),
    (6, 5, 21, 30, 0, 3, 1),
    (7, 16, 12, 9, 4, 8192, 0),
    (8, 4, 60, 40, 6, 4112, 0),
    (9, 8, 7, 200, 2, 8, 8),
    (10, 6, 1, 500, 3, 1, 0),
    (11, 2, 200, 8, 40, 64, 0),
    # 16-byte multiples under 1 KiB: the most whole rows in 4 KiB (48, 112,
    # 272, 400, 720, 1008 B), tiles of whole 128-byte lines on 256 threads
    # (688 B) and on 128 threads (832 B), each over several tiles per run
    (12, 4, 30, 60, 2, 48, 0),
    (13, 8, 20, 40, 3, 112, 0),
    (14, 4, 25, 30, 1, 272, 0),
    (15, 2, 40, 20, 4, 400, 0),
    (16, 4, 15, 25, 0, 688, 0),
    (17, 8, 10, 15, 2, 720, 0),
    (18, 4, 12, 20, 1, 832, 0),
    (19, 2, 18, 30, 3, 1008, 0),
]


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[f"seed{c[0]}" for c in RANDOM_CASES])
def test_random_swap_parity(thd, case):
    import torch
    seed, cp, docs, max_chunk, n_empty, rb, offset = case
    w = W.random_packed(seed, cp, docs, max_chunk, n_empty, row_shape=(rb,), row_dtype="uint8")
    cu, total = w.cu_padded, w.total
    say("random", case, "T", total, "slots", w.n_slots)
    route = build(thd, cu, cp, total)
    check_route_matches_oracle(route, cu, cp, total)
    x_host = w.rows_host()
    nbytes = total * rb
    in_buf = torch.empty(nbytes + 64, dtype=torch.uint8, device="cuda")
    out_buf = torch.full((nbytes + 64,), 0xCD, dtype=torch.uint8, device="cuda")
    in_buf[offset:offset + nbytes] = torch.from_numpy(x_host.reshape(-1)).cuda()
    for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
        out_buf.fill_(0xCD)
        code = thd.thd_swap(route.handle, d, in_buf.data_ptr() + offset, out_buf.data_ptr() + offset, total, rb)
        assert code == thd.THD_OK
        torch.cuda.synchronize()
        got = out_buf.cpu().numpy()
        want = O.swap_rows(x_host, cu, cp, total, direction).reshape(-1)
        assert np.array_equal(got[offset:offset + nbytes], want), direction
        # guard bands on both sides stay untouched
        assert (got[:offset] == 0xCD).all() and (got[offset + nbytes:] == 0xCD).all()


@pytest.mark.parametrize("tile_bytes,nt,block,order,rb", [
    (1, 1, 256, 1, 48), (1, 0, 512, 2, 48), (1 << 20, 1, 1024, 1, 48), (4096, 0, 128, 2, 48),
    (20000, 1, 512, 1, 4096), (20000, 0, 1024, 2, 4096), (1000, 1, 128, 2, 4096),
    (3 * 4096, 1, 256, 1, 4096), (0, 1, 0, 0, 8192), (0, 0, 0, 0, 8208),
    (0, 1, 0, 0, 4096), (0, 1, 0, 2, 2048), (5000, 1, 0, 2, 36),
    (0, 1, 0, 0, 8), (0, 1, 0, 0, 1), (0, 0, 0, 0, 16), (0, 1, 0, 0, 2),
    (4096, 1, 128, 64, 4096), (8192, 1, 512, 3, 8192), (0, 1, 0, 1 << 30, 8192), (0, 1, 0, 7, 48),
    # rows cut into slices (tile_bytes below the row size)
    (4096, 1, 128, 1, 8192), (2048, 1, 128, 64, 8192), (3000, 0, 256, 1, 8208), (16, 1, 128, 5, 4096),
    # the built-in shape on row sizes between and beyond the measured ones
    (0, 1, 0, 0, 6144), (0, 1, 0, 0, 4112), (0, 1, 0, 0, 12288), (0, 1, 0, 0, 65536),
    (0, 1, 0, 0, 10000),
])
def test_launch_shapes_do_not_change_results(thd, tile_bytes, nt, block, order, rb):
    import torch
    w = W.random_packed(42, 4, 30, 60, 3, row_shape=(rb,), row_dtype="uint8")
    cu, total = w.cu_padded, w.total
    say("launch shape", tile_bytes, nt, block, order, rb, "T", total)
    route = build(thd, cu, 4, total)
    x = torch.from_numpy(w.rows_host()).cuda()
    thd.thd_route_launch_shape(route.handle, tile_bytes, nt, block, order)
    out = route.swap(x, thd.Z2C)
    back = route.swap(out, thd.C2Z)
    torch.cuda.synchronize()
    want = O.swap_rows(w.rows_host(), cu, 4, total, "z2c")
    assert np.array_equal(out.cpu().numpy(), want)
    assert torch.equal(back, x)


def test_launch_shape_belongs_to_its_route(thd):
    # an override on one route leaves another route of the same batch on the
    # built-in shape; its field checks run on the host
    import torch
    w = W.random_packed(43, 4, 20, 40, 2, row_shape=(4096,), row_dtype="uint8")
    cu, total = w.cu_padded, w.total
    say("launch shape per route, T", total)
    a = build(thd, cu, 4, total)
    b = build(thd, cu, 4, total)
    for bad in ((-1, 1, 0, 0), (0, 2, 0, 0), (0, -1, 0, 0), (0, 1, 300, 0), (0, 1, 0, -1)):
        with pytest.raises(thd.ThdError):
            thd.thd_route_launch_shape(a.handle, *bad)
    thd.thd_route_launch_shape(a.handle, 1000, 0, 512, 3)
    x = torch.from_numpy(w.rows_host()).cuda()
    out_a = a.swap(x, thd.Z2C)
    out_b = b.swap(x, thd.Z2C)
    torch.cuda.synchronize()
    want = O.swap_rows(w.rows_host(), cu, 4, total, "z2c")
    assert np.array_equal(out_a.cpu().numpy(), want)
    assert np.array_equal(out_b.cpu().numpy(), want)
    thd.thd_route_launch_shape(a.handle)  # back to the built-in shape
    assert torch.equal(a.swap(x, thd.Z2C), out_b)


# ---- label shift / MTP roll / valid mask ----

ROLL_CASES = [
    # seed, docs, max_chunk, empty, pad_max, max_shift, fill
    (0, 5, 4, 0, 0, 1, 0),
    (1, 40, 30, 5, 7, 4, 0),
    (2, 300, 3, 20, 3, 8, -1),
    (3, 64, 100, 1, 50, 2, 7),
    (4, 1, 2000, 2, 1, 3, 0),
]


@pytest.mark.parametrize("case", ROLL_CASES, ids=[f"seed{c[0]}" for c in ROLL_CASES])
def test_roll_parity(thd, case):
    import torch
    seed, docs, max_chunk, n_empty, pad_max, j, fill = case
    w = W.random_packed(seed, 2, docs, max_chunk, n_empty, pad_max=pad_max)
    total = w.total
    ids = w.ids()
    say("roll", case, "T", total)
    shifted, mask, status = thd.roll_labels(dev_i64(ids), dev_i32(w.cu_padded), dev_i32(w.cu_real), j, fill)
    torch.cuda.synchronize()
    want_s, want_m = O.roll_labels(ids, w.cu_padded, w.cu_real, total, j, fill)
    assert int(status.item()) == 0
    assert np.array_equal(shifted.cpu().numpy(), want_s)
    assert np.array_equal(mask.cpu().numpy(), want_m)
    # without real boundaries: every slot is all real tokens
    shifted, mask, status = thd.roll_labels(dev_i64(ids), dev_i32(w.cu_padded), None, j, fill)
    torch.cuda.synchronize()
    want_s, want_m = O.roll_labels(ids, w.cu_padded, None, total, j, fill)
    assert np.array_equal(shifted.cpu().numpy(), want_s)
    assert np.array_equal(mask.cpu().numpy(), want_m)


def test_roll_many_slots_global_path(thd):
    # more boundaries than the kernel stages in LDS: the global-memory search path
    import torch
    w = W.random_packed(77, 1, 9000, 3, 500, pad_max=2)
    total = w.total
    assert w.n_slots + 1 > 4096
    ids = w.ids()
    say("roll global path", w.n_slots, total)
    shifted, mask, status = thd.roll_labels(dev_i64(ids), dev_i32(w.cu_padded), dev_i32(w.cu_real), 3, -5)
    torch.cuda.synchronize()
    want_s, want_m = O.roll_labels(ids, w.cu_padded, w.cu_real, total, 3, -5)
    assert int(status.item()) == 0
    assert np.array_equal(shifted.cpu().numpy(), want_s)
    assert np.array_equal(mask.cpu().numpy(), want_m)


def test_worked_example_on_gpu(thd, golden):
    # The page's packed stream of §3.4 through the device path: per-rank tokens
    # of §3.6 and the valid mask / count of §3.4 and §3.8.
    import torch
    g = golden("p3_worked_example.txt")
    cu_pad = [int(v) for v in g["cu_seqlens_padded"]]
    cu = [int(v) for v in g["cu_seqlens"]]
    stream = np.frombuffer("".join(g["tokens"]).encode(), dtype=np.uint8).copy()
    route = build(thd, cu_pad, 2, 16)
    z = route.swap(torch.from_numpy(stream).cuda().view(16, 1), thd.C2Z)
    got = z.cpu().numpy().reshape(-1).tobytes().decode()
    assert got[:8] == "".join(g["rank0_tokens"]) and got[8:] == "".join(g["rank1_tokens"])
    _, mask, status = thd.roll_labels(dev_i64(stream.astype(np.int64)), dev_i32(cu_pad), dev_i32(cu), 1, 0)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert mask[0].cpu().numpy().tolist() == [int(v) for v in g["valid_mask"]]
    assert int(mask[0].sum().item()) == int(g["valid_total"][0])


# ---- the slow paths of the route build: global scratch instead of LDS, and
#      directory windows with more runs than the kernel stages in LDS ----

@pytest.mark.parametrize("seed,cp,docs,max_chunk,n_empty", [
    (200, 2, 7000, 3, 1200),      # many slots, documents still in LDS (the closed form)
    (201, 128, 5, 3, 2),          # cp 128: a 64 KiB split matrix in LDS
    (202, 2, 3000, 1, 0),         # 4-token documents: one-row runs through the closed form's directory tables
    (203, 3, 2500, 1, 40),
    (204, 2, 14000, 2, 300),      # 3 * n_slots words above the LDS budget: global scratch, then the
                                  # directory launch with thousands of runs per 4096-row window
    (205, 256, 4, 2, 1),          # cp^2 above the LDS budget: global scratch
    (206, 1024, 3, 2, 1),         # cp at THD_MAX_CP: a 4 MiB split matrix in global scratch
    (207, 128, 80, 1, 4),         # cp above the closed form's 64, too many segments for the one-launch
                                  # build: one workgroup with the route in LDS, then the directory launch
    (208, 64, 300, 2, 10),        # cp 64, the closed form's largest: 63 borders fill its border tables
    (209, 65, 300, 1, 3),         # cp 65, just past it: one workgroup with the route in LDS
])
def test_route_build_slow_paths(thd, seed, cp, docs, max_chunk, n_empty):
    import torch
    w = W.random_packed(seed, cp, docs, max_chunk, n_empty, row_shape=(20,), row_dtype="uint8")
    cu, total = w.cu_padded, w.total
    say("slow path", seed, cp, "slots", w.n_slots, "T", total)
    route = build(thd, cu, cp, total)
    check_route_matches_oracle(route, cu, cp, total)
    x = torch.from_numpy(w.rows_host()).cuda()
    for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
        out = route.swap(x, d)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), O.swap_rows(w.rows_host(), cu, cp, total, direction)), direction


@pytest.mark.parametrize("seed,cp,rb", [(300, 2, 8), (301, 3, 1), (302, 3, 8), (303, 5, 4), (304, 2, 16)])
def test_small_rows_with_dense_runs(thd, seed, cp, rb):
    # One-unit rows through the LDS-staged small-row path, on batches of
    # 2*cp-token documents whose runs are so short that some tiles overflow
    # the staged run window and take the piecewise fallback.
    import torch
    w = W.random_packed(seed, cp, 4000, 1, 50, row_shape=(rb,), row_dtype="uint8")
    cu, total = w.cu_padded, w.total
    say("small rows", seed, cp, rb, "T", total)
    route = build(thd, cu, cp, total)
    x = torch.from_numpy(w.rows_host()).cuda()
    for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
        out = route.swap(x, d)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), O.swap_rows(w.rows_host(), cu, cp, total, direction)), direction


@pytest.mark.parametrize("rb", [1, 2, 4, 8, 16])
def test_one_unit_rows_with_long_runs(thd, rb):
    # Rows of exactly one copy unit whose runs are longer than a tile of the
    # piecewise path: thd_swap and thd_swap_batch stream them as flat copies
    # instead of the LDS-staged path.  A short-document batch through the same
    # calls keeps the staged path.  Both against the oracle, byte for byte.
    import torch
    cp = 2
    for lens in ([65536, 40000, 32768 + 4, 4, 100000], [8, 12, 4] * 300):
        cu = W.cumulative(lens)
        total = int(cu[-1])
        say("one-unit rows", rb, "T", total, "slots", len(lens))
        route = thd.Route(len(lens), cp, total)
        route.build(dev_i32(cu), cp, total)
        hosts = [np.random.default_rng([rb, total, i]).integers(0, 256, (total, rb), dtype=np.uint8) for i in range(3)]
        ins = [torch.from_numpy(h).cuda() for h in hosts]
        for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
            wants = [O.swap_rows(h, cu, cp, total, direction) for h in hosts]
            out = route.swap(ins[0], d)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), wants[0]), (rb, total, direction)
            outs = [torch.empty_like(t) for t in ins]
            assert thd.thd_swap_batch(route.handle, d, ins, outs, [rb] * 3, total) == thd.THD_OK
            torch.cuda.synchronize()
            for k in range(3):
                assert np.array_equal(outs[k].cpu().numpy(), wants[k]), (rb, total, direction, k)
        route.close()


@pytest.mark.parametrize("nbytes,offset", [(1 << 20, 0), (1 << 20, 16), (4096 * 3 + 128, 0), (4096 * 37 + 16, 0),
                                           (1000, 8), (999, 4), (4098, 2), (12345, 1), (3, 0)])
def test_plain_copy(thd, nbytes, offset):
    # The calibration copy: every unit width (16/8/4/2/1 B from the size and
    # the pointers' alignment), 16-byte tiles of whole 128-byte lines (stored
    # through L2) and tiles that are not (an output 16 bytes off a line, a
    # last tile of one line, a ragged last tile); the guard bytes around the
    # destination must stay untouched.
    import torch
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device="cuda")
    say("copy", nbytes, offset)
    assert thd.thd_copy(src[offset:offset + nbytes], dst[offset:offset + nbytes], nbytes) == thd.THD_OK
    torch.cuda.synchronize()
    assert torch.equal(dst[offset:offset + nbytes], src[offset:offset + nbytes])
    assert (dst[:offset] == 7).all() and (dst[offset + nbytes:] == 7).all()


@pytest.mark.parametrize("nwords", [1, 127, 128, 129, 255, 256, 257, 256 * 37 + 5, 1 << 18])
def test_read_and_write_streams(thd, nwords):
    # The two streaming ceilings.  Read: the key is planted at the first and
    # last word, at tile borders and at random places of a random buffer, and
    # the count must equal NumPy's count of equal 16-byte words (added to what
    # the counter held).  Write: word w = four copies of w ^ seed, guard words
    # around the destination untouched.  Ragged last tiles throughout.
    import torch
    nbytes = 16 * nwords
    g = torch.Generator(device="cuda").manual_seed(nwords)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    key = bytes(range(7, 23))
    rng = np.random.default_rng(nwords)
    spots = {0, nwords - 1, min(nwords - 1, 255), min(nwords - 1, 256), min(nwords - 1, 127)}
    spots |= set(rng.integers(0, nwords, size=min(nwords, 9)).tolist())
    kt = torch.tensor(list(key), dtype=torch.uint8, device="cuda")
    for w in spots:
        src[16 * w:16 * w + 16] = kt
    count = torch.tensor([5], dtype=torch.int32, device="cuda")
    say("read stream", nwords)
    assert thd.thd_read_stream(src, nbytes, key, count) == thd.THD_OK
    words = src.cpu().numpy().reshape(-1, 16)
    expect = int((words == np.frombuffer(key, np.uint8)).all(axis=1).sum())
    assert expect >= len(spots)
    assert int(count.item()) == 5 + expect

    seed = 0x9E3779B9
    dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device="cuda")
    say("write stream", nwords)
    assert thd.thd_write_stream(dst[32:32 + nbytes], nbytes, seed) == thd.THD_OK
    got = dst.cpu().numpy()
    w = (np.arange(nwords, dtype=np.uint64) & 0xFFFFFFFF).astype(np.uint32) ^ np.uint32(seed)
    assert np.array_equal(got[32:32 + nbytes].view(np.uint32).reshape(-1, 4), np.repeat(w[:, None], 4, axis=1))
    assert (got[:32] == 7).all() and (got[32 + nbytes:] == 7).all()


@pytest.mark.parametrize("seed,cp,docs,max_chunk,n_empty,rb", [
    (400, 4, 290, 2, 10, 8),      # ~2400 segments: the one-launch build writes the directory
    (401, 16, 60, 3, 4, 4096),    # cp 16, many directory workgroups, 4 KiB rows
    (402, 2, 700, 3, 20, 1),      # cp 2 near the fused limit, one-byte rows
    (403, 4, 490, 2, 10, 8),      # ~4000 segments: too many runs for LDS, build + directory kernels
    (404, 8, 60, 40, 3, 16),      # long chunks: few runs, two directory workgroups
    (405, 4, 200, 100, 5, 8),     # mixed runs over five directory workgroups
])
def test_route_build_with_and_without_fused_directory(thd, seed, cp, docs, max_chunk, n_empty, rb):
    # Batches on both sides of the one-launch build's limits (runs of both
    # orders held in LDS); dense short runs make every directory entry count.
    import torch
    w = W.random_packed(seed, cp, docs, max_chunk, n_empty, row_shape=(rb,), row_dtype="uint8")
    cu, total = w.cu_padded, w.total
    say("fused directory", seed, cp, "slots", w.n_slots, "T", total, "rb", rb)
    route = build(thd, cu, cp, total)
    check_route_matches_oracle(route, cu, cp, total)
    x = torch.from_numpy(w.rows_host()).cuda()
    for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
        out = route.swap(x, d)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), O.swap_rows(w.rows_host(), cu, cp, total, direction)), direction
