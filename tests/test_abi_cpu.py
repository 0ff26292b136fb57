"""The C-ABI library loads on the host and exports what include/*.h declare.

CPU only: nothing here launches a kernel.  The error paths called below are the
ones the library rejects on the host before any HIP call.
"""

import ctypes
import os
import re

import pytest

from conftest import ROOT

INCLUDE = os.path.join(ROOT, "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


def header_text():
    return "\n".join(open(h, encoding="utf-8").read() for h in HEADERS)


def declared_functions():
    text = re.sub(r"/\*.*?\*/", " ", header_text(), flags=re.S)
    names = re.findall(r"\b(?:int64_t|int|void|const char\s*\*)\s+(thd_[a-z_]+)\s*\(", text)
    return sorted(set(names))


def declared_constants():
    return {m.group(1): int(m.group(2))
            for m in re.finditer(r"#define\s+(THD_[A-Z0-9_]+)\s+(-?\d+)", header_text())}


@pytest.fixture(scope="module")
def pkg():
    import context_packed_sequence_amd as p
    return p


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("thd_build_route", "thd_swap", "thd_roll_labels"):
        assert n in names
    assert len(names) >= 10


def test_library_exports_every_declared_symbol(pkg):
    lib = pkg.binding.library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(pkg.EXPORTS) == set(declared_functions())


def test_binding_constants_match_header(pkg):
    for name, value in declared_constants().items():
        assert getattr(pkg.binding, name) == value, name


def test_strerror_covers_every_code(pkg):
    for name, value in declared_constants().items():
        if name.startswith("THD_ERR_") or name in ("THD_OK", "THD_IDENTITY"):
            assert pkg.thd_strerror(value) != "unknown code", name
    assert pkg.thd_strerror(12345) == "unknown code"


def test_host_rejections_without_device_work(pkg):
    lib = pkg.binding.library()
    h = ctypes.c_void_p()
    # bad create arguments are rejected before any HIP call
    assert lib.thd_route_create(0, 2, 16, ctypes.byref(h)) == pkg.THD_ERR_ARG
    assert lib.thd_route_create(4, 0, 16, ctypes.byref(h)) == pkg.THD_ERR_ARG
    assert lib.thd_route_create(4, pkg.THD_MAX_CP + 1, 16, ctypes.byref(h)) == pkg.THD_ERR_ARG
    assert lib.thd_route_create(4, 2, 2 ** 31, ctypes.byref(h)) == pkg.THD_ERR_ARG
    assert lib.thd_route_create(4, 2, 16, None) == pkg.THD_ERR_ARG
    # null route
    assert lib.thd_build_route(None, 1, 1, 2, 8, None) == pkg.THD_ERR_ARG
    assert lib.thd_swap(None, 0, 1, 2, 8, 4, None) == pkg.THD_ERR_ARG
    n = ctypes.c_int32()
    assert lib.thd_route_status(None, None, ctypes.byref(n)) == pkg.THD_ERR_ARG
    assert lib.thd_route_copy_out(None, None, ctypes.byref(n), 0, None, None, None) == pkg.THD_ERR_ARG
    assert lib.thd_route_info(None, None, None, None, None) == pkg.THD_ERR_ARG
    # roll: shift out of range, null boundaries, overlapping outputs
    assert lib.thd_roll_labels(8, 16, None, 1, 8, 0, 0, 4096, 8192, None, None) == pkg.THD_ERR_ARG
    assert lib.thd_roll_labels(8, 16, None, 1, 8, 9, 0, 4096, 8192, None, None) == pkg.THD_ERR_ARG
    assert lib.thd_roll_labels(8, None, None, 1, 8, 1, 0, 4096, 8192, None, None) == pkg.THD_ERR_ARG
    assert lib.thd_roll_labels(4096, 16, None, 1, 8, 1, 0, 4096 + 8, 1 << 20, None, None) == pkg.THD_ERR_ALIAS
    assert lib.thd_roll_labels(1 << 20, 16, None, 1, 8, 2, 0, 4096, 4096 + 64, None, None) == pkg.THD_ERR_ALIAS
    # pack: bad sizes, alignment, ids, workspace, overlapping outputs
    ws = lib.thd_pack_workspace_bytes(2, 8)
    assert ws > 0 and lib.thd_pack_workspace_bytes(-1, 8) == -1
    good = dict(tokens=1 << 20, batch=2, seq=8, pad=0, eod=1, align=4, cap=16, max_docs=4, fill=0,
                ws=1 << 24, ws_bytes=ws, packed=1 << 28, cu=1 << 30, cup=1 << 31, status=None)

    def pack(**kw):
        a = dict(good, **kw)
        return lib.thd_pack(a["tokens"], a["batch"], a["seq"], a["pad"], a["eod"], a["align"], a["cap"],
                            a["max_docs"], a["fill"], a["ws"], a["ws_bytes"], a["packed"], a["cu"], a["cup"],
                            a["status"], None)
    assert pack(align=0) == pkg.THD_ERR_ARG
    assert pack(cap=18) == pkg.THD_ERR_ARG
    assert pack(eod=0) == pkg.THD_ERR_ARG
    assert pack(ws_bytes=ws - 1) == pkg.THD_ERR_ARG
    assert pack(batch=-1) == pkg.THD_ERR_ARG
    assert pack(seq=pkg.THD_PACK_MAX_SEQ + 1) == pkg.THD_ERR_ARG
    assert lib.thd_pack_workspace_bytes(1, pkg.THD_PACK_MAX_SEQ + 1) == -1
    assert pack(cu=(1 << 31) + 8) == pkg.THD_ERR_ALIAS
    assert pack(packed=(1 << 20) + 64) == pkg.THD_ERR_ALIAS
    # plain copy: negative size, null pointers, overlap; zero bytes launches nothing
    assert lib.thd_copy(1 << 20, 1 << 24, -1, None) == pkg.THD_ERR_ARG
    assert lib.thd_copy(None, 1 << 24, 16, None) == pkg.THD_ERR_ARG
    assert lib.thd_copy(1 << 20, (1 << 20) + 8, 16, None) == pkg.THD_ERR_ALIAS
    assert lib.thd_copy(None, None, 0, None) == pkg.THD_OK
    # read and write streams: size a multiple of 16, aligned pointers, no overlap
    key = ctypes.create_string_buffer(16)
    assert lib.thd_read_stream(1 << 20, 24, key, 1 << 24, None) == pkg.THD_ERR_ARG
    assert lib.thd_read_stream(1 << 20, -16, key, 1 << 24, None) == pkg.THD_ERR_ARG
    assert lib.thd_read_stream((1 << 20) + 8, 16, key, 1 << 24, None) == pkg.THD_ERR_ARG
    assert lib.thd_read_stream(1 << 20, 16, key, None, None) == pkg.THD_ERR_ARG
    assert lib.thd_read_stream(1 << 20, 16, None, 1 << 24, None) == pkg.THD_ERR_ARG
    assert lib.thd_read_stream(1 << 20, 16, key, (1 << 24) + 2, None) == pkg.THD_ERR_ARG
    assert lib.thd_read_stream(1 << 20, 32768, key, (1 << 20) + 32764, None) == pkg.THD_ERR_ALIAS
    assert lib.thd_read_stream(None, 0, None, None, None) == pkg.THD_OK
    assert lib.thd_write_stream(1 << 20, 24, 0, None) == pkg.THD_ERR_ARG
    assert lib.thd_write_stream((1 << 20) + 4, 16, 0, None) == pkg.THD_ERR_ARG
    assert lib.thd_write_stream(None, 16, 0, None) == pkg.THD_ERR_ARG
    assert lib.thd_write_stream(None, 0, 0, None) == pkg.THD_OK
    # the launch-shape override belongs to a route: none given, nothing set
    assert lib.thd_route_launch_shape(None, 0, 1, 0, 0) == pkg.THD_ERR_ARG
    # the pack without allocation: bad sizes, and batches beyond its static
    # scratch, are refused on the host before the scratch is looked up
    def pack_noalloc(batch, seq):
        return lib.thd_pack_noalloc(None, batch, seq, 0, 1, 8, 8, 1, 0, None, None, None, None, None)
    assert pack_noalloc(-1, 8) == pkg.THD_ERR_ARG
    assert pack_noalloc(1, pkg.THD_PACK_MAX_SEQ + 1) == pkg.THD_ERR_ARG
    seq = 1024
    while lib.thd_pack_workspace_bytes(2, seq + 1024) <= pkg.THD_PACK_STATIC_BYTES:
        seq += 1024
    assert seq * 2 > 20_000_000                      # the limit admits about 24 million tokens
    assert pack_noalloc(2, seq + 1024) == pkg.THD_ERR_CAPACITY


def test_package_and_oracle_share_no_code():
    # The oracle imports nothing from the package and vice versa.
    pkg_dir = os.path.join(ROOT, "context_packed_sequence_amd")
    for d, other in ((os.path.join(ROOT, "oracle"), "context_packed_sequence_amd"), (pkg_dir, "oracle")):
        for f in os.listdir(d):
            if f.endswith(".py"):
                src = open(os.path.join(d, f), encoding="utf-8").read()
                assert not re.search(rf"^\s*(from|import)\s+{other}\b", src, flags=re.M), (d, f)


def test_wrappers_reject_wrong_buffers_before_any_device_call(pkg):
    # The C ABI sees bare pointers; the Python wrappers check dtypes and sizes
    # first, so a wrongly typed or short buffer never reaches a kernel.
    import torch
    cu = torch.tensor([0, 4, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="ids must be torch.int64"):
        pkg.roll_labels(torch.zeros(8, dtype=torch.int32), cu)
    with pytest.raises(ValueError, match="cu_seqlens_padded must be torch.int32"):
        pkg.roll_labels(torch.zeros(8, dtype=torch.int64), cu.long())
    with pytest.raises(ValueError, match="cu_seqlens must have 3 elements"):
        pkg.roll_labels(torch.zeros(8, dtype=torch.int64), cu, torch.tensor([0, 4], dtype=torch.int32))
    with pytest.raises(ValueError, match="tokens must be torch.int64"):
        pkg.pack(torch.zeros((2, 4), dtype=torch.int32), 0, 1, 4, 16, 4)
    with pytest.raises(ValueError, match="must be contiguous"):
        pkg.pack(torch.zeros((4, 2), dtype=torch.int64).t(), 0, 1, 4, 16, 4)
