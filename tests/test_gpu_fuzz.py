"""Seeded random sweeps on the GPU against the CPU oracle, byte for byte.

Many small batches drawn from one seeded generator, each through one device
call and compared whole with the oracle: cp from 1 to 64, 1-80 documents with
chunks of 1-64 tokens, empty slots anywhere, rows of 1-10240 bytes at byte
offsets that force every copy unit (16/8/4/2/1 B), both directions; the same
under random launch-shape overrides (tile size, cache policy, block size,
tile order); several tensors through one launch; label rolls with
real lengths shorter than the padded ones, in natural and in zigzag order;
packs of token rows with budgets that fit, that hold too few documents, too
few tokens, or both; corrupted boundary lists on every route-build path; and
route builds alone, cp up to 1024 and up to ~700 documents, on every build
path.  Each case is printed before it
runs, and every assertion names its case.
"""

import os

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import CODE_OF_KIND, check_route_matches_oracle, dev_i32, dev_i64, oracle_source_rows, say

pytestmark = pytest.mark.gpu

ROW_BYTES = [1, 2, 3, 4, 6, 8, 12, 16, 20, 32, 48, 64, 100, 256, 272, 400, 720, 1000, 1008, 1152, 1536, 2000, 2560,
             3584, 4096, 4112, 10240]
# THD_FUZZ_SCALE multiplies the case count of every sweep but the route builds
# (THD_FUZZ_ROUTES sets that one); the first cases stay the same.
SCALE = max(1, int(os.environ.get("THD_FUZZ_SCALE", "1")))
CPS = [1, 2, 3, 4, 5, 6, 8, 12, 16, 32, 64]
OFFSETS = [0, 0, 0, 1, 2, 4, 8]


@pytest.fixture(scope="module")
def thd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import context_packed_sequence_amd as thd
    return thd


def draw_batch(rng, cp, max_tokens):
    docs = int(rng.integers(1, 81))
    max_chunk = int(rng.integers(1, 65))
    while docs > 1 and 2 * cp * max_chunk * docs > 2 * max_tokens:
        docs = max(1, docs // 2)
        max_chunk = max(1, max_chunk // 2)
    while max_chunk > 1 and 2 * cp * max_chunk > 2 * max_tokens:
        max_chunk //= 2
    return docs, max_chunk, int(rng.integers(0, 11))


def test_fuzz_swap(thd):
    import torch
    rng = np.random.default_rng([W.BASE_SEED, 900])
    for case in range(160 * SCALE):
        cp = int(rng.choice(CPS))
        rb = int(rng.choice(ROW_BYTES))
        offset = int(rng.choice(OFFSETS))
        docs, max_chunk, n_empty = draw_batch(rng, cp, 200000 // max(rb, 16))
        w = W.random_packed([901, case], cp, docs, max_chunk, n_empty, row_shape=(rb,), row_dtype="uint8")
        total = w.total
        tag = f"swap case {case}: cp {cp} docs {docs} chunk<={max_chunk} empty {n_empty} rb {rb} off {offset} T {total}"
        say(tag)
        route = thd.Route(max(1, w.n_slots), cp, max(total, 1))
        route.build(dev_i32(w.cu_padded), cp, total)
        assert route.status() == 0, tag
        x_host = w.rows_host()
        nbytes = total * rb
        in_buf = torch.empty(nbytes + 64, dtype=torch.uint8, device="cuda")
        out_buf = torch.empty(nbytes + 64, dtype=torch.uint8, device="cuda")
        in_buf[offset:offset + nbytes] = torch.from_numpy(x_host.reshape(-1)).cuda()
        for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
            out_buf.fill_(0xA5)
            code = thd.thd_swap(route.handle, d, in_buf.data_ptr() + offset, out_buf.data_ptr() + offset, total, rb)
            torch.cuda.synchronize()
            got = out_buf.cpu().numpy()
            if cp == 1:
                assert code == thd.THD_IDENTITY, tag
                assert (got == 0xA5).all(), tag  # nothing written
                continue
            assert code == thd.THD_OK, tag
            want = O.swap_rows(x_host, w.cu_padded, cp, total, direction).reshape(-1)
            assert np.array_equal(got[offset:offset + nbytes], want), f"{tag} {direction}"
            assert (got[:offset] == 0xA5).all() and (got[offset + nbytes:] == 0xA5).all(), f"{tag} {direction}"
        route.close()


TUNE_TILE = [0, 1, 16, 100, 512, 1000, 4096, 5000, 16384, 65536]
TUNE_BLOCK = [0, 128, 256, 512, 1024]
TUNE_ORDER = [0, 1, 2, 5, 64, 128, 100000]


def test_fuzz_route_build(thd):
    # Route builds alone, many of them: cp from 2 to 1024, up to ~700
    # documents of 2cp-64*2cp tokens and 30 empty slots, so every build path
    # (run slots in closed form over many workgroups, one launch in LDS, LDS
    # plus the directory kernel, the workspace in global memory) is drawn;
    # chunks of one token put the closed form's directory tables at their
    # reach (a 16-row block spanning 16 one-row segments).  Runs in both orders and the split matrix must
    # equal the oracle's, and a swap of row-stamped 16-byte rows in each
    # direction must fetch the rows the oracle names.  THD_FUZZ_ROUTES sets
    # the number of cases (default 300; one-off runs of 20000 passed).
    import torch
    n_cases = int(os.environ.get("THD_FUZZ_ROUTES", "300"))
    rng = np.random.default_rng([W.BASE_SEED, 4242])
    cps = [2, 3, 4, 5, 6, 8, 12, 16, 24, 32, 64, 128, 256, 512, 1024]
    for case in range(n_cases):
        cp = int(rng.choice(cps))
        docs = int(rng.integers(1, 700))
        max_chunk = int(rng.choice([1, 2, 3, 8, 16, 64]))
        while 2 * cp * max_chunk * docs > 600000 and docs > 1:
            docs = max(1, docs // 2)
        n_empty = int(rng.integers(0, 30))
        w = W.random_packed([4243, case], cp, docs, max_chunk, n_empty, row_shape=(16,), row_dtype="uint8")
        total = w.total
        tag = f"route case {case}: cp {cp} docs {docs} chunk<={max_chunk} empty {n_empty} T {total}"
        say(tag)
        route = thd.Route(max(1, w.n_slots), cp, max(total, 1))
        route.build(dev_i32(w.cu_padded), cp, total)
        r = check_route_matches_oracle(route, w.cu_padded, cp, total)
        if total > 0:
            x = torch.arange(total, dtype=torch.int64, device="cuda").repeat_interleave(2).view(total, 2)
            for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
                got = route.swap(x, d)[:, 0].cpu().numpy()
                assert np.array_equal(got, oracle_source_rows(r, direction)), f"{tag} {direction}"
        route.close()


def test_fuzz_swap_launch_shapes(thd):
    # every launch-shape override (tile size, cache policy, block size, tile
    # order) on rows of any size at byte offsets that force every copy unit:
    # the result never depends on the shape
    import torch
    rng = np.random.default_rng([W.BASE_SEED, 930])
    for case in range(200 * SCALE):
        cp = int(rng.choice(CPS[1:]))
        rb = int(rng.choice(ROW_BYTES)) if rng.random() < 0.6 else int(rng.integers(1, 9001))
        offset = int(rng.choice(OFFSETS + [3, 6, 12]))
        tune = (int(rng.choice(TUNE_TILE)), int(rng.integers(0, 2)), int(rng.choice(TUNE_BLOCK)),
                int(rng.choice(TUNE_ORDER)))
        docs, max_chunk, n_empty = draw_batch(rng, cp, max(1, (2 << 20) // rb))
        w = W.random_packed([931, case], cp, docs, max_chunk, n_empty, row_shape=(1,), row_dtype="uint8")
        total = w.total
        tag = f"shape case {case}: cp {cp} rb {rb} off {offset} T {total} slots {w.n_slots} tuning {tune}"
        say(tag)
        route = thd.Route(max(1, w.n_slots), cp, max(total, 1))
        route.build(dev_i32(w.cu_padded), cp, total)
        x_host = np.random.default_rng([932, case]).integers(0, 256, (total, rb), dtype=np.uint8)
        nbytes = total * rb
        in_buf = torch.empty(nbytes + 64, dtype=torch.uint8, device="cuda")
        out_buf = torch.empty(nbytes + 64, dtype=torch.uint8, device="cuda")
        in_buf[offset:offset + nbytes] = torch.from_numpy(x_host.reshape(-1)).cuda()
        thd.thd_route_launch_shape(route.handle, *tune)
        for direction, d in (("z2c", thd.Z2C), ("c2z", thd.C2Z)):
            out_buf.fill_(0xA5)
            code = thd.thd_swap(route.handle, d, in_buf.data_ptr() + offset, out_buf.data_ptr() + offset, total,
                                rb)
            torch.cuda.synchronize()
            assert code == thd.THD_OK, tag
            got = out_buf.cpu().numpy()
            want = O.swap_rows(x_host, w.cu_padded, cp, total, direction).reshape(-1)
            assert np.array_equal(got[offset:offset + nbytes], want), f"{tag} {direction}"
            assert (got[:offset] == 0xA5).all() and (got[offset + nbytes:] == 0xA5).all(), f"{tag} {direction}"
        route.close()


def test_fuzz_swap_batch(thd):
    import torch
    rng = np.random.default_rng([W.BASE_SEED, 910])
    for case in range(50 * SCALE):
        cp = int(rng.choice(CPS[1:]))
        docs, max_chunk, n_empty = draw_batch(rng, cp, 8000)
        w = W.random_packed([911, case], cp, docs, max_chunk, n_empty, row_shape=(1,), row_dtype="uint8")
        total = w.total
        n = int(rng.integers(1, 7))
        rbs = [int(rng.choice(ROW_BYTES[:-2])) for _ in range(n)]
        direction = ["z2c", "c2z"][int(rng.integers(0, 2))]
        tag = f"batch case {case}: cp {cp} T {total} row bytes {rbs} {direction}"
        say(tag)
        route = thd.Route(max(1, w.n_slots), cp, max(total, 1))
        route.build(dev_i32(w.cu_padded), cp, total)
        hosts = [np.random.default_rng([912, case, i]).integers(0, 256, (total, rb), dtype=np.uint8)
                 for i, rb in enumerate(rbs)]
        # every tensor at its own byte offset inside a larger buffer, so the
        # copy unit and the realigning copy's head and tail vary per tensor;
        # the bytes around each output must stay untouched
        in_offs = [int(v) for v in rng.integers(0, 16, n)]
        out_offs = [int(v) for v in rng.integers(0, 16, n)]
        ins, outs, out_bufs = [], [], []
        for h, rb, io, oo in zip(hosts, rbs, in_offs, out_offs):
            nbytes = total * rb
            ib = torch.empty(nbytes + 32, dtype=torch.uint8, device="cuda")
            ib[io:io + nbytes] = torch.from_numpy(h.reshape(-1)).cuda()
            ins.append(ib[io:io + nbytes].view(total, rb))
            ob = torch.full((nbytes + 32,), 0x5A, dtype=torch.uint8, device="cuda")
            out_bufs.append(ob)
            outs.append(ob[oo:oo + nbytes].view(total, rb))
        tag += f" offsets in {in_offs} out {out_offs}"
        code = thd.thd_swap_batch(route.handle, thd.Z2C if direction == "z2c" else thd.C2Z, ins, outs, rbs, total)
        assert code == thd.THD_OK, tag
        torch.cuda.synchronize()
        for i, (h, o, ob, oo) in enumerate(zip(hosts, outs, out_bufs, out_offs)):
            assert np.array_equal(o.cpu().numpy(), O.swap_rows(h, w.cu_padded, cp, total, direction)), f"{tag} #{i}"
            b = ob.cpu().numpy()
            assert (b[:oo] == 0x5A).all() and (b[oo + o.numel():] == 0x5A).all(), f"{tag} #{i} guard"
        route.close()


def test_fuzz_roll(thd):
    import torch
    rng = np.random.default_rng([W.BASE_SEED, 920])
    for case in range(60 * SCALE):
        cp = int(rng.choice(CPS[1:9]))
        docs, max_chunk, n_empty = draw_batch(rng, cp, 20000)
        pad_max = int(rng.integers(0, 2 * cp * max_chunk + 1))
        j = int(rng.integers(1, 9))
        fill = int(rng.integers(-3, 4))
        w = W.random_packed([921, case], cp, docs, max_chunk, n_empty, pad_max=pad_max)
        total = w.total
        tag = f"roll case {case}: cp {cp} T {total} slots {w.n_slots} pad<={pad_max} shifts {j} fill {fill}"
        say(tag)
        ids = w.ids()
        want_s, want_m = O.roll_labels(ids, w.cu_padded, w.cu_real, total, j, fill)
        shifted, mask, status = thd.roll_labels(dev_i64(ids), dev_i32(w.cu_padded), dev_i32(w.cu_real), j, fill)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, tag
        assert np.array_equal(shifted.cpu().numpy(), want_s), tag
        assert np.array_equal(mask.cpu().numpy(), want_m), tag
        # the same roll written in zigzag order: the natural-order result sliced
        # to zigzag rows by the oracle's c->z swap
        route = thd.Route(max(1, w.n_slots), cp, max(total, 1))
        route.build(dev_i32(w.cu_padded), cp, total)
        shifted, mask, status = route.roll_labels_zigzag(dev_i64(ids), dev_i32(w.cu_padded), dev_i32(w.cu_real), j,
                                                         fill)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, tag
        for k in range(j):
            assert np.array_equal(shifted[k].cpu().numpy(),
                                  O.swap_rows(want_s[k], w.cu_padded, cp, total, "c2z")), f"{tag} shift {k + 1}"
        for k in range(j + 1):
            assert np.array_equal(mask[k].cpu().numpy(),
                                  O.swap_rows(want_m[k], w.cu_padded, cp, total, "c2z")), f"{tag} mask {k}"
        route.close()


def test_fuzz_pack(thd):
    import torch
    pad, eod = 0, 1
    codes = dict(CODE_OF_KIND, PACK_DOCS=thd.THD_ERR_PACK_DOCS, PACK_CAPACITY=thd.THD_ERR_PACK_CAPACITY)
    rng = np.random.default_rng([W.BASE_SEED, 940])
    for case in range(120 * SCALE):
        batch = int(rng.integers(1, 41))
        seq = int(rng.integers(1, min(5000, 40000 // batch) + 1))
        eod_rate = float(rng.choice([0.0, 0.001, 0.01, 0.05, 0.3]))
        tail = [None, 0, 1, 10, seq][int(rng.integers(0, 5))]
        inner = float(rng.choice([0.0, 0.01, 0.1]))
        align = int(rng.choice([1, 2, 3, 4, 8, 16, 64, 512]))
        rows = W.token_rows([941, case], batch, seq, pad, eod, eod_rate, tail, inner)
        # the budget is a host-side choice, sized from the oracle's documents
        _, cu_r, _ = O.pack_batch(rows, pad, eod, 1, batch * seq, batch * seq + 1, 0)
        lengths = np.diff(cu_r.astype(np.int64))
        n_docs = int(np.count_nonzero(lengths > 0))
        used = int(sum(n + (-n) % align for n in lengths[:n_docs]))
        kind = rng.choice(["fits", "fits", "fits", "docs", "capacity", "both"])
        capacity = used + align * int(rng.choice([0, 1, 7]))
        max_docs = n_docs + int(rng.choice([0, 1, 5]))
        if kind in ("docs", "both") and n_docs > 0:
            max_docs = n_docs - 1
        if kind in ("capacity", "both") and used >= align:
            capacity = used - align * int(rng.integers(1, min(3, used // align) + 1))
        fill = int(rng.integers(-5, 5))
        tag = f"pack case {case}: [{batch}, {seq}] eod {eod_rate} align {align} docs {n_docs} used {used} " \
              f"capacity {capacity} max_docs {max_docs}"
        say(tag)
        try:
            want, want_code = O.pack_batch(rows, pad, eod, align, capacity, max_docs, fill), 0
        except O.OracleInputError as e:
            want, want_code = None, codes[e.kind]
        nbytes = thd.thd_pack_workspace_bytes(batch, seq)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        packed = torch.full((capacity,), -7, dtype=torch.int64, device="cuda")
        cu_real = torch.full((max_docs + 2,), -7, dtype=torch.int32, device="cuda")
        cu_pad = torch.full((max_docs + 2,), -7, dtype=torch.int32, device="cuda")
        status = torch.full((1,), 99, dtype=torch.int32, device="cuda")
        assert thd.thd_pack(dev_i64(rows), batch, seq, pad, eod, align, capacity, max_docs, fill, ws, nbytes, packed,
                            cu_real, cu_pad, status) == thd.THD_OK, tag
        torch.cuda.synchronize()
        assert int(status.item()) == want_code, tag
        if want is None:
            assert (packed == -7).all() and (cu_real == -7).all() and (cu_pad == -7).all(), tag
        else:
            assert np.array_equal(packed.cpu().numpy(), want[0]), tag
            assert np.array_equal(cu_real.cpu().numpy(), want[1]), tag
            assert np.array_equal(cu_pad.cpu().numpy(), want[2]), tag


def test_fuzz_bad_boundaries(thd):
    # one to three corruptions of a valid boundary list (first boundary,
    # a decrease, the total, a length off the 2*cp grid), with cp and slot
    # counts that take each build path (one launch; closed-form runs, with or
    # without the directory launch; one workgroup in LDS, at cp 128; one
    # workgroup in global memory): the status is the oracle's first failing
    # rule and no swap writes anything
    import torch
    rng = np.random.default_rng([W.BASE_SEED, 950])
    for case in range(60 * SCALE):
        cp = int(rng.choice([2, 3, 4, 8, 16, 64, 128]))
        n_docs = int(rng.choice([3, 100, 1500, 14000]))
        max_chunk = max(1, min(8, 120000 // (2 * cp * n_docs)))
        w = W.random_packed([951, case], cp, n_docs, max_chunk, int(rng.integers(0, 4)), row_shape=(1,),
                            row_dtype="uint8")
        cu = w.cu_padded.astype(np.int64).copy()
        total = int(cu[-1])
        n = len(cu) - 1
        kinds = rng.choice(["start", "monotone", "total", "divisible"], size=int(rng.integers(1, 4)), replace=False)
        for kind in kinds:
            if kind == "start":
                cu[0] = int(rng.choice([-3, -1, 1, 2, 2 * cp]))
            elif kind == "monotone" and n >= 2:
                i = int(rng.integers(1, n))
                cu[i] = cu[i - 1] - int(rng.integers(1, 10))
            elif kind == "total":
                total += 2 * cp * int(rng.integers(1, 4))
            elif kind == "divisible":
                room = [i for i in range(1, n) if cu[i + 1] - cu[i] >= 2 * cp and cu[i] >= cu[i - 1]]
                if room:
                    i = room[int(rng.integers(0, len(room)))]
                    cu[i] += int(rng.integers(1, 2 * cp))
        try:
            O.build_route(cu.tolist(), cp, total)
            continue                               # the corruptions cancelled out: nothing to check
        except O.OracleInputError as e:
            rule = e.kind
        want = CODE_OF_KIND[rule]
        tag = f"bad boundaries case {case}: cp {cp} slots {n} T {total} corruptions {list(kinds)} -> {rule}"
        say(tag)
        route = thd.Route(n, cp, total)
        route.build(dev_i32(cu), cp, total)
        assert route.status() == want, tag
        x = torch.arange(total * 4, dtype=torch.int32, device="cuda").view(total, 4)
        out = torch.full_like(x, -77)
        for d in (thd.Z2C, thd.C2Z):
            assert thd.thd_swap(route.handle, d, x, out, total, 16) == thd.THD_OK, tag
        torch.cuda.synchronize()
        assert (out == -77).all(), tag
        by_src, _, _ = route.copy_out()
        assert by_src.shape[0] == 0, tag
        route.close()
